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


def test_mla_full_size_sampled():
    log("mla full: generating")
    inp = make_config_inputs("mla_deepseek_v2")[0]
    dev = Dev(inp)
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
