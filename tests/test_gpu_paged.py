"""GPU parity of kv_append_paged and decode_attn_paged against the fp64 oracle.

Inputs come from the seeded generator; the oracle sees the same stored values.
Append is compared bit for bit over the whole cache buffers; attention
outputs elementwise within the contract tolerance (tests/contract.py).
"""

import zlib

import numpy as np
import pytest
import torch

import oracle
from contract import assert_contract
from gpu_util import Paged, down_bits, down_f64, log, up
from workloads import make_config_inputs, make_paged_decode, UNUSED_TABLE_ENTRY

pytestmark = pytest.mark.gpu

kvd = pytest.importorskip("kv_cache_decode_02_amd")


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _oracle_out(inp):
    return oracle.decode_attn_paged(inp.q, inp.k_pool, inp.v_pool, inp.block_table,
                                    inp.seq_lens, inp.dtype, inp.k_new, inp.v_new)


def _run_step(dev, partition=0, scale=None):
    kvd.kv_append_paged(dev.k_cache, dev.v_cache, dev.k_new, dev.v_new, dev.table, dev.seq)
    out = kvd.decode_attn_paged(dev.q, dev.k_cache, dev.v_cache, dev.table, dev.seq,
                                dev.inp.max_seq_len, scale=scale, partition_tokens=partition)
    torch.cuda.synchronize()
    return out


# --- append -----------------------------------------------------------------

APPEND_CASES = [
    ("bf16-gqa", dict(B=5, H_q=32, H_kv=8, d=128, lens=[1, 16, 17, 500, 4096], dtype="bf16")),
    ("f32-tiny", dict(B=1, H_q=4, H_kv=4, d=32, lens=[129], dtype="f32")),
    ("bf16-mha-d64", dict(B=3, H_q=4, H_kv=4, d=64, lens=[32, 33, 2], dtype="bf16")),
]


@pytest.mark.parametrize("name,c", APPEND_CASES, ids=[n for n, _ in APPEND_CASES])
def test_append_bit_exact(name, c):
    log(f"append {name}")
    inp = make_paged_decode(np.random.default_rng(100), c["B"], c["H_q"], c["H_kv"], c["d"],
                            c["lens"], dtype=c["dtype"])
    dev = Paged(inp)
    kvd.kv_append_paged(dev.k_cache, dev.v_cache, dev.k_new, dev.v_new, dev.table, dev.seq)
    torch.cuda.synchronize()
    k_ref, v_ref = oracle.append_paged(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new,
                                       inp.block_table, inp.seq_lens)
    assert np.array_equal(down_bits(dev.k_cache).view(np.uint8), k_ref.view(np.uint8))
    assert np.array_equal(down_bits(dev.v_cache).view(np.uint8), v_ref.view(np.uint8))


def test_append_latent_cache_without_v():
    log("append latent")
    rng = np.random.default_rng(101)
    lens = [4096, 1, 77]
    B, w = len(lens), 576
    nb = sum(-(-n // 16) for n in lens)
    table = np.full((B, 256), UNUSED_TABLE_ENTRY, dtype=np.int32)
    perm = rng.permutation(nb).astype(np.int32)
    pos = 0
    for b, n in enumerate(lens):
        table[b, :-(-n // 16)] = perm[pos:pos - (-n // 16)]
        pos += -(-n // 16)
    pool = rng.integers(0, 2**16, size=(nb, 16, 1, w), dtype=np.uint16)
    new = rng.integers(0, 2**16, size=(B, 1, w), dtype=np.uint16)
    c_dev = up(pool)
    kvd.kv_append_paged(c_dev, None, up(new), None, up(table), up(np.array(lens, np.int32)))
    torch.cuda.synchronize()
    ref, _ = oracle.append_paged(pool, None, new, None, table, np.array(lens))
    assert np.array_equal(down_bits(c_dev), ref)


# --- decode attention ----------------------------------------------------------

DECODE_CASES = [
    ("mha-ragged", dict(B=3, H_q=32, H_kv=32, d=128, lens=[4096, 1000, 17], pt=0)),
    ("gqa-r4-edges", dict(B=8, H_q=32, H_kv=8, d=128, lens=[1, 15, 16, 17, 511, 512, 513, 3000], pt=256)),
    ("long-r8-split512", dict(B=2, H_q=64, H_kv=8, d=128, lens=[5000, 2049], pt=512)),
    ("mqa-r8-pt64", dict(B=3, H_q=8, H_kv=1, d=128, lens=[100, 700, 2000], pt=64)),
    ("r16-two-chunks-d64", dict(B=2, H_q=16, H_kv=1, d=64, lens=[300, 1200], pt=128)),
    ("r2-d32-pt16", dict(B=2, H_q=8, H_kv=4, d=32, lens=[33, 999], pt=16)),
    ("pt1024", dict(B=2, H_q=8, H_kv=2, d=128, lens=[1025, 2500], pt=1024)),
    ("identity-table", dict(B=2, H_q=16, H_kv=4, d=128, lens=[64, 333], pt=0, table="identity")),
    ("f32-d128", dict(B=2, H_q=4, H_kv=2, d=128, lens=[77, 640], pt=0, dtype="f32")),
    ("f32-d64-r8", dict(B=2, H_q=16, H_kv=2, d=64, lens=[5, 1500], pt=0, dtype="f32")),
    ("f32-d32-r1", dict(B=3, H_q=4, H_kv=4, d=32, lens=[1, 129, 130], pt=0, dtype="f32")),
    # the largest group (64 query heads on one K/V head: 16 wavefronts of 4 heads)
    ("r64-mqa", dict(B=2, H_q=64, H_kv=1, d=128, lens=[700, 33], pt=0)),
    # groups of 12: three 4-head wavefronts per K/V head, two idle wavefronts per
    # 8-wave workgroup
    ("r12-balanced", dict(B=3, H_q=24, H_kv=2, d=64, lens=[257, 40, 1600], pt=0)),
    ("r12-split256", dict(B=3, H_q=24, H_kv=2, d=64, lens=[257, 40, 1600], pt=256)),
    # head_dim 32 with groups of 4 and 8 (MFMA flavour), a group of 24 (the
    # VALU flavour: more than 16 heads and not a multiple of 16)
    ("r4-d32", dict(B=3, H_q=8, H_kv=2, d=32, lens=[1, 300, 1025], pt=0)),
    ("r8-d32-pt64", dict(B=2, H_q=16, H_kv=2, d=32, lens=[70, 513], pt=64)),
    ("r24-valu", dict(B=2, H_q=48, H_kv=2, d=128, lens=[900, 33], pt=0)),
]


@pytest.mark.parametrize("name,c", DECODE_CASES, ids=[n for n, _ in DECODE_CASES])
def test_decode_parity(name, c):
    log(f"decode {name}")
    inp = make_paged_decode(np.random.default_rng(zlib.crc32(name.encode())), c["B"], c["H_q"],
                            c["H_kv"], c["d"], c["lens"], dtype=c.get("dtype", "bf16"),
                            table=c.get("table", "permuted"))
    dev = Paged(inp)
    out = _run_step(dev, c["pt"])
    rep = assert_contract(down_f64(out), _oracle_out(inp), name)
    log(f"  max_err {rep['max_err']:.3e} scaled {rep['scaled']:.3e}")


@pytest.mark.parametrize("name,c", DECODE_CASES, ids=[n for n, _ in DECODE_CASES])
def test_fused_append_parity(name, c):
    # decode_attn_paged_append = kv_append_paged + decode_attn_paged in one pass: the
    # caches afterwards equal the oracle's append bit for bit, the output meets the
    # contract against the oracle (the new slot holds the NaN sentinel before the
    # call, so reading it instead of k_new / v_new would show).
    log(f"fused append {name}")
    inp = make_paged_decode(np.random.default_rng(zlib.crc32(name.encode()) + 1), c["B"],
                            c["H_q"], c["H_kv"], c["d"], c["lens"], dtype=c.get("dtype", "bf16"),
                            table=c.get("table", "permuted"))
    dev = Paged(inp)
    out = kvd.decode_attn_paged_append(dev.q, dev.k_cache, dev.v_cache, dev.k_new, dev.v_new,
                                       dev.table, dev.seq, inp.max_seq_len,
                                       partition_tokens=c["pt"])
    torch.cuda.synchronize()
    k_ref, v_ref = oracle.append_paged(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new,
                                       inp.block_table, inp.seq_lens)
    assert np.array_equal(down_bits(dev.k_cache).view(np.uint8), k_ref.view(np.uint8))
    assert np.array_equal(down_bits(dev.v_cache).view(np.uint8), v_ref.view(np.uint8))
    rep = assert_contract(down_f64(out), _oracle_out(inp), name)
    log(f"  max_err {rep['max_err']:.3e} scaled {rep['scaled']:.3e}")


def test_tiny_config_both_layers():
    for layer, inp in enumerate(make_config_inputs("tiny")):
        log(f"tiny layer {layer}")
        dev = Paged(inp)
        out = _run_step(dev)
        rep = assert_contract(down_f64(out), _oracle_out(inp), f"tiny layer {layer}")
        # fp32 storage and arithmetic: far inside the contract
        assert rep["max_err"] < 1e-5, rep


def test_phases_equal_single_call():
    log("partials + merge")
    inp = make_paged_decode(np.random.default_rng(7), 4, 32, 8, 128, [900, 40, 2049, 16])
    dev = Paged(inp)
    one = _run_step(dev, 256)
    ws = kvd.alloc_workspace(inp.B, 32, 8, 128, inp.max_seq_len, 256)
    kvd.decode_attn_paged_partials(dev.q, dev.k_cache, dev.v_cache, dev.table, dev.seq,
                                   inp.max_seq_len, ws, partition_tokens=256)
    two = torch.empty_like(dev.q)
    kvd.decode_attn_merge(two, dev.seq, 8, inp.max_seq_len, ws, partition_tokens=256)
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int16), two.view(torch.int16))


SPLIT_CASES = [
    ("gqa-r4", dict(B=5, H_q=32, H_kv=8, d=128, lens=[4096, 40, 17, 1000, 300], dtype="bf16")),
    ("mha-d64", dict(B=3, H_q=16, H_kv=16, d=64, lens=[2000, 33, 700], dtype="bf16")),
    ("r2-f32", dict(B=3, H_q=8, H_kv=4, d=128, lens=[1500, 16, 2], dtype="f32")),
    ("r8-two-chunks", dict(B=2, H_q=64, H_kv=8, d=128, lens=[3000, 100], dtype="bf16")),
]


@pytest.mark.parametrize("name,c", SPLIT_CASES, ids=[n for n, _ in SPLIT_CASES])
def test_balanced_split_with_an_empty_sequence(name, c):
    # Balanced split (automatic mode) with sequence 1 at length 0 between
    # sequences cut into many pieces: the empty one gets zeros, the others
    # meet the contract, and the one-call path equals partials + merge.
    log(f"balanced split {name}")
    inp = make_paged_decode(np.random.default_rng(zlib.crc32(name.encode()) + 2), c["B"],
                            c["H_q"], c["H_kv"], c["d"], c["lens"], dtype=c["dtype"])
    dev = Paged(inp)
    kvd.kv_append_paged(dev.k_cache, dev.v_cache, dev.k_new, dev.v_new, dev.table, dev.seq)
    seq = dev.seq.clone()
    seq[1] = 0
    L = inp.max_seq_len
    one = kvd.decode_attn_paged(dev.q, dev.k_cache, dev.v_cache, dev.table, seq, L)
    ws = kvd.alloc_workspace(inp.B, c["H_q"], c["H_kv"], c["d"], L)
    kvd.decode_attn_paged_partials(dev.q, dev.k_cache, dev.v_cache, dev.table, seq, L, ws)
    two = torch.empty_like(dev.q)
    kvd.decode_attn_merge(two, seq, c["H_kv"], L, ws)
    torch.cuda.synchronize()
    iv = torch.int16 if c["dtype"] == "bf16" else torch.int32
    assert torch.equal(one.view(iv), two.view(iv))
    assert torch.count_nonzero(one[1]).item() == 0
    keep = [b for b in range(inp.B) if b != 1]  # the others do not see sequence 1
    assert_contract(down_f64(one)[keep], _oracle_out(inp)[keep], name)


def test_workspace_serves_calls_of_any_size():
    # One workspace, sized for the largest call and never cleared, used by
    # calls of different batch, heads and lengths in turn (the data of one
    # call lands where the next keeps other data): each output equals that of
    # a fresh workspace.
    log("workspace reuse")
    shapes = [(6, 32, 8, 128, [4096, 1, 900, 2000, 64, 3000]), (2, 8, 2, 64, [700, 33]),
              (3, 64, 8, 128, [1500, 4000, 16]), (6, 32, 8, 128, [100, 4096, 17, 18, 2500, 5])]
    need = max(kvd.decode_attn_workspace_bytes(B, hq, hkv, d, max(lens), 0)
               for B, hq, hkv, d, lens in shapes)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")  # garbage to start
    for i, (B, hq, hkv, d, lens) in enumerate(shapes):
        inp = make_paged_decode(np.random.default_rng(40 + i), B, hq, hkv, d, lens)
        dev = Paged(inp)
        kvd.kv_append_paged(dev.k_cache, dev.v_cache, dev.k_new, dev.v_new, dev.table, dev.seq)
        got = kvd.decode_attn_paged(dev.q, dev.k_cache, dev.v_cache, dev.table, dev.seq,
                                    inp.max_seq_len, workspace=ws)
        fresh = kvd.decode_attn_paged(dev.q, dev.k_cache, dev.v_cache, dev.table, dev.seq,
                                      inp.max_seq_len)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), fresh.view(torch.int16)), i
    assert_contract(down_f64(got), _oracle_out(inp), "last reused call")


def test_block_placement_is_bit_identical():
    log("placement")
    a = make_paged_decode(np.random.default_rng(8), 3, 32, 8, 128, [700, 33, 1600])
    perm = np.random.default_rng(9).permutation(a.num_blocks).astype(np.int32)
    b_table = np.where(a.block_table == UNUSED_TABLE_ENTRY, UNUSED_TABLE_ENTRY,
                       perm[np.minimum(a.block_table, a.num_blocks - 1)])
    k_pool, v_pool = np.empty_like(a.k_pool), np.empty_like(a.v_pool)
    k_pool[perm] = a.k_pool
    v_pool[perm] = a.v_pool
    outs = []
    for table, kp, vp in ((a.block_table, a.k_pool, a.v_pool), (b_table, k_pool, v_pool)):
        kc, vc, tb = up(kp), up(vp), up(table)
        seq = up(a.seq_lens)
        kvd.kv_append_paged(kc, vc, up(a.k_new), up(a.v_new), tb, seq)
        outs.append(kvd.decode_attn_paged(up(a.q), kc, vc, tb, seq, a.max_seq_len))
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


def test_scale_argument():
    log("scale")
    inp = make_paged_decode(np.random.default_rng(10), 2, 8, 2, 64, [300, 45])
    dev = Paged(inp)
    out = _run_step(dev, 0, scale=0.5)
    ref = oracle.decode_attn_paged(inp.q, inp.k_pool, inp.v_pool, inp.block_table,
                                   inp.seq_lens, "bf16", inp.k_new, inp.v_new, scale=0.5)
    assert_contract(down_f64(out), ref, "scale 0.5")


def test_zero_length_gives_zeros_and_bad_entries_are_skipped():
    log("degenerate lengths / entries")
    inp = make_paged_decode(np.random.default_rng(11), 3, 8, 2, 128, [40, 40, 40])
    dev = Paged(inp)
    kvd.kv_append_paged(dev.k_cache, dev.v_cache, dev.k_new, dev.v_new, dev.table, dev.seq)
    # sequence 0 claims length 0; sequence 2's second block id points outside the pool
    seq = dev.seq.clone()
    seq[0] = 0
    table = dev.table.clone()
    table[2, 1] = inp.num_blocks + 5
    out = kvd.decode_attn_paged(dev.q, dev.k_cache, dev.v_cache, table, seq, 40)
    torch.cuda.synchronize()
    got = down_f64(out)
    assert np.all(got[0] == 0)
    k2, v2 = oracle.append_paged(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new,
                                 inp.block_table, inp.seq_lens)
    ref1 = oracle.decode_attn_paged(inp.q[1:2], k2, v2, inp.block_table[1:2], [40], "bf16")
    assert_contract(got[1:2], ref1, "untouched sequence")
    # positions 16..31 of sequence 2 are skipped: attention over the rest
    rows = [t for t in range(40) if not 16 <= t < 32]
    K = oracle.to_f64(oracle.gather_logical(k2, inp.block_table, 2, 40), "bf16")[rows]
    V = oracle.to_f64(oracle.gather_logical(v2, inp.block_table, 2, 40), "bf16")[rows]
    ref2 = oracle.decode_attention(oracle.to_f64(inp.q[2], "bf16"), K, V)
    assert_contract(got[2], ref2, "skipped block")


def test_empty_batch_is_a_no_op():
    q = torch.empty((0, 8, 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((1, 16, 2, 128), dtype=torch.bfloat16, device="cuda")
    table = torch.zeros((0, 1), dtype=torch.int32, device="cuda")
    seq = torch.zeros((0,), dtype=torch.int32, device="cuda")
    out = kvd.decode_attn_paged(q, kc, kc.clone(), table, seq, 16)
    assert out.shape == (0, 8, 128)


@pytest.mark.parametrize("B", [8191, 8193])
def test_batch_around_the_balanced_split_limit(B):
    # The automatic mode splits batches of up to 8191 sequences evenly (their
    # prefix sums fill 64 KiB of LDS) and larger ones in fixed partitions.
    # Both sides of the limit, checked on a sample of sequences (each
    # sequence's output depends on its own rows only).
    log(f"batch {B}")
    rng = np.random.default_rng(B)
    lens = rng.integers(1, 49, size=B)
    inp = make_paged_decode(rng, B, 8, 2, 64, lens)
    dev = Paged(inp)
    got = down_f64(_run_step(dev, 0))
    sel = np.unique(np.concatenate([[0, B - 1], rng.integers(0, B, size=62)]))
    ref = oracle.decode_attn_paged(inp.q[sel], inp.k_pool, inp.v_pool, inp.block_table[sel],
                                   inp.seq_lens[sel], inp.dtype, inp.k_new[sel], inp.v_new[sel])
    rep = assert_contract(got[sel], ref, f"batch {B}")
    log(f"  {len(sel)} sequences, max_err {rep['max_err']:.3e}")


# --- full-size workloads, sampled -----------------------------------------------

FULL = [("mha_llama2_7b", 0), ("gqa_llama3_8b", 0), ("long_gqa_split", 512)]


@pytest.mark.parametrize("name,pt", FULL, ids=[n for n, _ in FULL])
def test_full_size_sampled(name, pt):
    log(f"full {name}: generating")
    inp = make_config_inputs(name)[0]
    dev = Paged(inp)
    log(f"full {name}: running (kv bytes {inp.kv_bytes_read / 1e9:.2f} GB)")
    out = _run_step(dev, pt)
    got = down_f64(out)
    assert np.all(np.isfinite(got))
    # any size: each output is a convex combination of V rows of its group
    r = inp.H_q // inp.H_kv
    rng = np.random.default_rng(1)
    picks = [(0, 0), (inp.B - 1, inp.H_kv - 1)] + [
        (int(rng.integers(inp.B)), int(rng.integers(inp.H_kv))) for _ in range(4)]
    log(f"full {name}: oracle on {len(picks)} (sequence, kv head) samples")
    for b, g in picks:
        n = int(inp.seq_lens[b])
        Kh = oracle.gather_history(inp.k_pool[:, :, g:g + 1], inp.block_table, inp.seq_lens, b)
        Vh = oracle.gather_history(inp.v_pool[:, :, g:g + 1], inp.block_table, inp.seq_lens, b)
        K = np.concatenate([oracle.to_f64(Kh, "bf16"), oracle.to_f64(inp.k_new[b:b + 1, g:g + 1], "bf16")])
        V = np.concatenate([oracle.to_f64(Vh, "bf16"), oracle.to_f64(inp.v_new[b:b + 1, g:g + 1], "bf16")])
        assert K.shape[0] == n
        q = oracle.to_f64(inp.q[b, g * r:(g + 1) * r], "bf16")
        ref = oracle.decode_attention(q, K, V)
        assert_contract(got[b, g * r:(g + 1) * r], ref, f"{name} b={b} g={g}")
        vmax = np.abs(V).max()
        assert np.all(np.abs(got[b, g * r:(g + 1) * r]) <= vmax * (1 + 1e-2))
    log(f"full {name}: ok")
