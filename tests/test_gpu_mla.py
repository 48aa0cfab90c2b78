"""GPU parity of decode_attn_mla (absorbed MLA over a latent cache) with the
fp64 oracle.  Inputs: the seeded generator's latent cache and queries (std
1/24 as the DeepSeek-V2-shaped workload, and a unit-variance variant so that
the tolerance is not vacuous for small outputs)."""

import zlib

import numpy as np
import pytest
import torch

import oracle
from contract import assert_contract
from gpu_util import down_f64, log, up
from workloads import make_config_inputs, make_mla, UNUSED_TABLE_ENTRY

pytestmark = pytest.mark.gpu

kvd = pytest.importorskip("kv_cache_decode_02_amd")


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


class Dev:
    def __init__(self, inp):
        self.inp = inp
        self.q = up(inp.q)
        self.c = up(inp.c_pool)
        self.c_new = up(inp.c_new[:, None, :])
        self.table = up(inp.block_table)
        self.seq = up(inp.seq_lens)


def _step(dev, pt=0, scale=None):
    kvd.kv_append_paged(dev.c[:, :, None, :], None, dev.c_new, None, dev.table, dev.seq)
    out = kvd.decode_attn_mla(dev.q, dev.c, dev.table, dev.seq, dev.inp.max_seq_len,
                              scale=scale, partition_tokens=pt)
    torch.cuda.synchronize()
    return out


def _ref(inp, scale=None):
    scale = kvd.mla_default_scale() if scale is None else scale
    return oracle.mla_decode_paged(inp.q, inp.c_pool, inp.block_table, inp.seq_lens, inp.d_c,
                                   scale, c_new=inp.c_new)


CASES = [
    ("h128-ragged-std24", dict(B=3, H=128, lens=[1, 33, 700], std=1 / 24, pt=0)),
    ("h128-unit-var", dict(B=3, H=128, lens=[17, 64, 1000], std=1.0, pt=64)),
    ("h16-one-wave", dict(B=2, H=16, lens=[31, 500], std=1.0, pt=32)),
    ("h64-pt256", dict(B=2, H=64, lens=[256, 257], std=0.5, pt=256)),
    ("h80-partial-group", dict(B=2, H=80, lens=[90, 300], std=1.0, pt=0)),
    # The second 32-head block of a 64-head group half filled, then empty.
    ("h48-half-block", dict(B=2, H=48, lens=[129, 1024], std=1.0, pt=96)),
    ("h32-one-block", dict(B=3, H=32, lens=[2, 95, 640], std=1.0, pt=0)),
    # Many 32-token tiles per partition (odd and even counts), long rows.
    ("h128-long-odd-tiles", dict(B=2, H=128, lens=[2015, 4096], std=1 / 24, pt=1024)),
]


@pytest.mark.parametrize("name,c", CASES, ids=[n for n, _ in CASES])
def test_mla_parity(name, c):
    log(f"mla {name}")
    inp = make_mla(np.random.default_rng(zlib.crc32(name.encode())), c["B"], c["H"], 512, 64,
                   c["lens"], std=c["std"])
    dev = Dev(inp)
    out = _step(dev, c["pt"])
    rep = assert_contract(down_f64(out), _ref(inp), name)
    log(f"  max_err {rep['max_err']:.3e} scaled {rep['scaled']:.3e}")


@pytest.mark.parametrize("name,c", CASES, ids=[n for n, _ in CASES])
def test_mla_fused_append(name, c):
    # decode_attn_mla_append = kv_append_paged + decode_attn_mla in one pass.
    # The new slot holds the NaN sentinel before the call, so reading it
    # instead of c_new would show.  Afterwards the cache equals the oracle's
    # append bit for bit, and the output equals the two separate calls bit for
    # bit (the row reaches the same LDS tile either way) and meets the
    # contract against the oracle.
    log(f"mla fused append {name}")
    inp = make_mla(np.random.default_rng(zlib.crc32(name.encode()) + 1), c["B"], c["H"], 512, 64,
                   c["lens"], std=c["std"])
    fused, sep = Dev(inp), Dev(inp)
    out = kvd.decode_attn_mla_append(fused.q, fused.c, fused.c_new[:, 0], fused.table, fused.seq,
                                     inp.max_seq_len, partition_tokens=c["pt"])
    torch.cuda.synchronize()
    ref_cache, _ = oracle.append_paged(inp.c_pool, None, inp.c_new, None, inp.block_table,
                                       inp.seq_lens)
    assert np.array_equal(fused.c.cpu().view(torch.int16).numpy().view(np.uint16), ref_cache)
    two = _step(sep, c["pt"])
    assert torch.equal(out.view(torch.int16), two.view(torch.int16))
    rep = assert_contract(down_f64(out), _ref(inp), name)
    log(f"  max_err {rep['max_err']:.3e} scaled {rep['scaled']:.3e}")


def test_mla_fused_append_phases_and_skipped_last_block():
    # The partials entry point with the merge equals the single call; a last
    # block outside the pool is neither written nor read (its positions get
    # no weight), as with the separate calls.
    inp = make_mla(np.random.default_rng(5), 3, 64, 512, 64, [300, 33, 1000], std=1.0)
    one_dev, two_dev = Dev(inp), Dev(inp)
    one = kvd.decode_attn_mla_append(one_dev.q, one_dev.c, one_dev.c_new[:, 0], one_dev.table,
                                     one_dev.seq, inp.max_seq_len, partition_tokens=256)
    ws = kvd.alloc_workspace(3, 64, 1, 512, inp.max_seq_len, 256)
    kvd.decode_attn_mla_append_partials(two_dev.q, two_dev.c, two_dev.c_new[:, 0], two_dev.table,
                                        two_dev.seq, inp.max_seq_len, ws, partition_tokens=256)
    two = torch.empty_like(one)
    kvd.decode_attn_merge(two, two_dev.seq, 1, inp.max_seq_len, ws, partition_tokens=256)
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int16), two.view(torch.int16))
    assert torch.equal(one_dev.c.view(torch.int16), two_dev.c.view(torch.int16))
    # sequence 1 (33 positions): its third block (positions 32..) is outside the pool
    dev = Dev(inp)
    table = dev.table.clone()
    table[1, 2] = inp.num_blocks + 7
    before = dev.c.clone()
    out = kvd.decode_attn_mla_append(dev.q, dev.c, dev.c_new[:, 0], table, dev.seq,
                                     inp.max_seq_len, partition_tokens=256)
    torch.cuda.synchronize()
    got = down_f64(out)
    scale = kvd.mla_default_scale()
    C = oracle.to_f64(oracle.gather_logical(inp.c_pool, inp.block_table, 1, 32), "bf16")
    assert_contract(got[1], oracle.mla_decode(oracle.to_f64(inp.q[1], "bf16"), C, 512, scale),
                    "skipped last block")
    # only the other two sequences' new slots changed
    # (bitwise: the unfilled slots hold NaN)
    changed = (dev.c.view(torch.int16) != before.view(torch.int16)).any(dim=-1).nonzero()
    slots = {(int(inp.block_table[b, (n - 1) // 16]), (n - 1) % 16) for b, n in ((0, 300), (2, 1000))}
    assert {(int(i), int(j)) for i, j in changed.cpu().numpy()} == slots


def test_mla_scale_and_skipped_block():
    log("mla scale / bad entry")
    inp = make_mla(np.random.default_rng(3), 2, 32, 512, 64, [100, 100], std=1.0)
    dev = Dev(inp)
    kvd.kv_append_paged(dev.c[:, :, None, :], None, dev.c_new, None, dev.table, dev.seq)
    table = dev.table.clone()
    table[1, 2] = inp.num_blocks + 3     # positions 32..47 of sequence 1 are skipped
    out = kvd.decode_attn_mla(dev.q, dev.c, table, dev.seq, 100, scale=0.05)
    torch.cuda.synchronize()
    got = down_f64(out)
    c2, _ = oracle.append_paged(inp.c_pool, None, inp.c_new, None, inp.block_table, inp.seq_lens)
    ref0 = oracle.mla_decode_paged(inp.q[:1], c2, inp.block_table[:1], [100], 512, 0.05)
    assert_contract(got[:1], ref0, "scale 0.05")
    rows = [t for t in range(100) if not 32 <= t < 48]
    C = oracle.to_f64(oracle.gather_logical(c2, inp.block_table, 1, 100), "bf16")[rows]
    ref1 = oracle.mla_decode(oracle.to_f64(inp.q[1], "bf16"), C, 512, 0.05)
    assert_contract(got[1], ref1, "skipped block")


def test_mla_phases_equal_single_call():
    inp = make_mla(np.random.default_rng(4), 2, 128, 512, 64, [300, 129], std=1 / 24)
    dev = Dev(inp)
    one = _step(dev, 64)
    ws = kvd.alloc_workspace(2, 128, 1, 512, inp.max_seq_len, 64)
    kvd.decode_attn_mla_partials(dev.q, dev.c, dev.table, dev.seq, inp.max_seq_len, ws,
                                 partition_tokens=64)
    two = torch.empty_like(one)
    kvd.decode_attn_merge(two, dev.seq, 1, inp.max_seq_len, ws, partition_tokens=64)
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int16), two.view(torch.int16))


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
def test_mla_full_size_sampled(fused):
    log(f"mla full ({'fused' if fused else 'separate'} append): generating")
    inp = make_config_inputs("mla_deepseek_v2")[0]
    dev = Dev(inp)
    if fused:
        out = kvd.decode_attn_mla_append(dev.q, dev.c, dev.c_new[:, 0], dev.table, dev.seq,
                                         inp.max_seq_len)
        torch.cuda.synchronize()
    else:
        out = _step(dev)
    got = down_f64(out)
    assert np.all(np.isfinite(got))
    scale = kvd.mla_default_scale()
    for b in (0, 17, inp.B - 1):
        C = np.concatenate([
            oracle.to_f64(oracle.gather_history(inp.c_pool, inp.block_table, inp.seq_lens, b), "bf16"),
            oracle.to_f64(inp.c_new[b:b + 1], "bf16")])
        ref = oracle.mla_decode(oracle.to_f64(inp.q[b], "bf16"), C, 512, scale)
        assert_contract(got[b], ref, f"mla full b={b}")
    log("mla full: ok")


def _bf16_bits(x):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def _plant(inp, b, rows):
    """rows: {position: z} -- the latent row of sequence b at that position
    becomes a multiple of query head 0's vector, so that head 0's score there
    is about z (log2 units, scale and log2(e) included) above that of a
    near-zero row.  The positions precede the appended one."""
    scale = kvd.mla_default_scale()
    q0 = oracle.to_f64(inp.q[b, 0], "bf16")
    unit = q0 / (scale * np.log2(np.e) * float(q0 @ q0))
    for t, z in rows.items():
        assert t < int(inp.seq_lens[b]) - 1
        blk = int(inp.block_table[b, t // 16])
        inp.c_pool[blk, t % 16] = _bf16_bits(oracle.to_f64(inp.c_pool[blk, t % 16], "bf16") +
                                            z * unit)


# Scores far above the first tile's maximum in a later tile of the same
# partition: up to 64 log2 units the weights stay in range in one pass; past
# that the partition runs a second time with the exact maximum.  A ramp moves
# head 0's scores up along the whole sequence (one partition of 1024 tokens:
# 150 log2 units from its first tile to its last).
SPREAD = [
    ("spike-40", 0, {0: {40: 40.0, 200: 40.0}, 1: {33: 40.0, 900: 40.0}}),
    ("spike-100", 64, {0: {40: 100.0, 250: 100.0}, 1: {70: 100.0, 999: 100.0}}),
    ("ramp-150", 1024, {0: {t: 150.0 * t / 511 for t in range(299)},
                     1: {t: 150.0 * (t % 512) / 511 for t in range(999)}}),
]


@pytest.mark.parametrize("name,pt,plants", SPREAD, ids=[n for n, _, _ in SPREAD])
def test_mla_score_spread(name, pt, plants):
    log(f"mla score spread {name}")
    inp = make_mla(np.random.default_rng(zlib.crc32(name.encode())), 2, 128, 512, 64,
                   [300, 1001], std=1 / 24)
    for b, rows in plants.items():
        _plant(inp, b, rows)
    fused, sep = Dev(inp), Dev(inp)
    out = kvd.decode_attn_mla_append(fused.q, fused.c, fused.c_new[:, 0], fused.table, fused.seq,
                                     inp.max_seq_len, partition_tokens=pt)
    two = _step(sep, pt)
    assert torch.equal(out.view(torch.int16), two.view(torch.int16))
    got = down_f64(out)
    assert np.all(np.isfinite(got))
    rep = assert_contract(got, _ref(inp), name)
    log(f"  max_err {rep['max_err']:.3e} scaled {rep['scaled']:.3e}")
