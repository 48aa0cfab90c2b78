"""GPU parity of the sliding-window decode against the fp64 oracle.

Table entries of blocks wholly before each row's window point at a block
filled with NaN: a kernel that read them would return NaN.
"""

import zlib

import numpy as np
import pytest
import torch

import oracle
from contract import assert_contract
from gpu_util import Paged, down_f64, log, up
from workloads import make_paged_decode

pytestmark = pytest.mark.gpu

kvd = pytest.importorskip("kv_cache_decode_02_amd")


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _stale_before_window(inp, window):
    """A copy of the inputs with one extra NaN block that every table entry
    wholly before the window points to."""
    nan = np.uint16(0x7FC0) if inp.dtype == "bf16" else np.float32(np.nan)
    k_pool = np.concatenate([inp.k_pool, np.full((1,) + inp.k_pool.shape[1:], nan)])
    v_pool = np.concatenate([inp.v_pool, np.full((1,) + inp.v_pool.shape[1:], nan)])
    table = inp.block_table.copy()
    for b, n in enumerate(inp.seq_lens):
        first = oracle.window_start(int(n), window) // 16
        table[b, :first] = inp.num_blocks
    return k_pool, v_pool, table


CASES = [
    ("gqa-mixed", dict(B=6, H_q=32, H_kv=8, d=128, lens=[1, 17, 300, 1000, 4096, 2049]), 0,
     [1, 15, 16, 17, 100, 1024, 5000]),
    ("gqa-pt256", dict(B=4, H_q=32, H_kv=8, d=128, lens=[40, 700, 3000, 513]), 256,
     [1, 33, 256, 600]),
    ("mha-d64", dict(B=3, H_q=4, H_kv=4, d=64, lens=[129, 2000, 64]), 0, [7, 64, 130]),
    ("f32-r2", dict(B=2, H_q=8, H_kv=4, d=128, lens=[77, 640], dtype="f32"), 64, [5, 100]),
]


@pytest.mark.parametrize("name,c,pt,windows", CASES, ids=[n for n, *_ in CASES])
def test_window_parity(name, c, pt, windows):
    inp = make_paged_decode(np.random.default_rng(zlib.crc32(name.encode()) + 5), c["B"],
                            c["H_q"], c["H_kv"], c["d"], c["lens"], dtype=c.get("dtype", "bf16"))
    for W in windows:
        log(f"window {name} W={W} pt={pt}")
        k_pool, v_pool, table = _stale_before_window(inp, W)
        kc, vc, tb, seq = up(k_pool), up(v_pool), up(table), up(inp.seq_lens)
        kvd.kv_append_paged(kc, vc, up(inp.k_new), up(inp.v_new), tb, seq)
        out = kvd.decode_attn_paged_window(up(inp.q), kc, vc, tb, seq, inp.max_seq_len, W,
                                           partition_tokens=pt)
        torch.cuda.synchronize()
        ref = oracle.decode_attn_paged_window(inp.q, k_pool, v_pool, table, inp.seq_lens,
                                              inp.dtype, W, inp.k_new, inp.v_new)
        assert_contract(down_f64(out), ref, f"{name} W={W}")


def test_window_covering_everything_equals_full_decode():
    log("window >= length")
    inp = make_paged_decode(np.random.default_rng(77), 3, 32, 8, 128, [100, 2000, 33])
    dev = Paged(inp)
    kvd.kv_append_paged(dev.k_cache, dev.v_cache, dev.k_new, dev.v_new, dev.table, dev.seq)
    full = kvd.decode_attn_paged(dev.q, dev.k_cache, dev.v_cache, dev.table, dev.seq,
                                 inp.max_seq_len)
    win = kvd.decode_attn_paged_window(dev.q, dev.k_cache, dev.v_cache, dev.table, dev.seq,
                                       inp.max_seq_len, inp.max_seq_len)
    torch.cuda.synchronize()
    assert torch.equal(full.view(torch.int16), win.view(torch.int16))


def test_merge_never_reads_rows_of_empty_pieces():
    # Fixed partitions wholly before the window are empty pieces (l = 0).
    # The merge gives them no weight and must not read their rows: with
    # those rows overwritten by NaN the output stays bit for bit the same.
    log("merge skips empty pieces")
    B, Hq, Hkv, d, pt, W = 4, 32, 8, 128, 256, 33
    inp = make_paged_decode(np.random.default_rng(91), B, Hq, Hkv, d, [40, 700, 3000, 513])
    dev = Paged(inp)
    kvd.kv_append_paged(dev.k_cache, dev.v_cache, dev.k_new, dev.v_new, dev.table, dev.seq)
    ws = kvd.alloc_workspace(B, Hq, Hkv, d, inp.max_seq_len, pt)
    kvd.decode_attn_paged_window_partials(dev.q, dev.k_cache, dev.v_cache, dev.table, dev.seq,
                                          inp.max_seq_len, W, ws, partition_tokens=pt)
    clean = torch.empty_like(dev.q)
    kvd.decode_attn_merge(clean, dev.seq, Hkv, inp.max_seq_len, ws, partition_tokens=pt)
    P = -(-inp.max_seq_len // pt)
    f = ws.view(torch.float32)
    o = f[:B * Hq * P * d].view(B * Hq * P, d)
    ml_at = -(-(B * Hq * P * d * 4) // 256) * 256 // 4
    ml = f[ml_at:ml_at + B * Hq * P * 2].view(B * Hq * P, 2)
    empty = ml[:, 1] == 0
    assert int(empty.sum()) > 0
    o[empty] = float("nan")
    poisoned = torch.empty_like(dev.q)
    kvd.decode_attn_merge(poisoned, dev.seq, Hkv, inp.max_seq_len, ws, partition_tokens=pt)
    torch.cuda.synchronize()
    assert torch.equal(clean.view(torch.int16), poisoned.view(torch.int16))
