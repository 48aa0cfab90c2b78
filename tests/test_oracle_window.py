"""Pins of the sliding-window decode oracle (CPU only).

The gathered-slice formulation is checked against a second one (the banded
causal score matrix of a full recompute), against full attention when the
window covers everything, against the single-token case, and against the
page's point that positions outside the window may be dropped: their
contents do not matter, those inside do.
"""

import numpy as np
import pytest

import oracle
from workloads import make_paged_decode


def _inputs(seed, lens, H_q=4, H_kv=2, d=16):
    return make_paged_decode(np.random.default_rng(seed), len(lens), H_q, H_kv, d, lens,
                             dtype="f32", sentinel="zero")


def _window(inp, W):
    return oracle.decode_attn_paged_window(inp.q, inp.k_pool, inp.v_pool, inp.block_table,
                                           inp.seq_lens, "f32", W, inp.k_new, inp.v_new)


def test_window_start():
    assert oracle.window_start(100, 30) == 70
    assert oracle.window_start(20, 30) == 0
    assert oracle.window_start(1, 1) == 0
    with pytest.raises(ValueError):
        oracle.window_start(5, 0)


def test_wide_window_is_full_attention():
    inp = _inputs(1, [40, 17, 1])
    full = oracle.decode_attn_paged(inp.q, inp.k_pool, inp.v_pool, inp.block_table,
                                    inp.seq_lens, "f32", inp.k_new, inp.v_new)
    assert np.array_equal(_window(inp, 40), full)
    assert np.array_equal(_window(inp, 10 ** 6), full)


def test_window_of_one_is_the_new_value():
    inp = _inputs(2, [40, 17, 1])
    out = _window(inp, 1)
    r = inp.H_q // inp.H_kv
    for b in range(inp.B):
        for h in range(inp.H_q):
            assert np.array_equal(out[b, h], inp.v_new[b, h // r].astype(np.float64))


def test_banded_causal_recompute_agrees():
    rng = np.random.default_rng(3)
    T, d, W = 50, 8, 13
    K = rng.standard_normal((T, d))
    V = rng.standard_normal((T, d))
    Q = rng.standard_normal((T, d))
    rows = oracle.causal_attention(Q, K, V, past_len=0, window=W)
    for i in (0, 5, 12, 13, 30, T - 1):
        lo = max(0, i + 1 - W)
        want = oracle.decode_attention(Q[i][None], K[lo:i + 1, None], V[lo:i + 1, None])[0]
        assert np.max(np.abs(rows[i] - want)) < 1e-12
    # the decode row is the last row of the banded matrix
    lens = np.array([T], np.int32)
    table = np.arange(-(-T // 16), dtype=np.int32)[None, :]
    pool = np.zeros((table.shape[1], 16, 1, d))
    vpool = np.zeros_like(pool)
    for t in range(T):
        pool[t // 16, t % 16, 0] = K[t]
        vpool[t // 16, t % 16, 0] = V[t]
    got = oracle.decode_attn_paged_window(Q[-1][None, None].astype(np.float32),
                                          pool.astype(np.float32), vpool.astype(np.float32),
                                          table, lens, "f32", W)
    assert np.max(np.abs(got[0, 0] - rows[-1])) < 1e-6


def test_rows_outside_the_window_do_not_matter():
    inp = _inputs(4, [70, 33])
    W = 20
    ref = _window(inp, W)
    rng = np.random.default_rng(5)
    k2, v2 = inp.k_pool.copy(), inp.v_pool.copy()
    inside = None
    for b, n in enumerate(inp.seq_lens):
        start = oracle.window_start(int(n), W)
        for t in range(start):
            blk, off = oracle.slot_of(inp.block_table, b, t)
            k2[blk, off] = rng.standard_normal(k2.shape[2:]) * 100
            v2[blk, off] = rng.standard_normal(v2.shape[2:]) * 100
        inside = oracle.slot_of(inp.block_table, b, start)
    same = oracle.decode_attn_paged_window(inp.q, k2, v2, inp.block_table, inp.seq_lens, "f32",
                                           W, inp.k_new, inp.v_new)
    assert np.array_equal(same, ref)
    v2[inside] += 1.0  # the oldest visible row of the last sequence
    moved = oracle.decode_attn_paged_window(inp.q, k2, v2, inp.block_table, inp.seq_lens, "f32",
                                            W, inp.k_new, inp.v_new)
    assert np.max(np.abs(moved[-1] - ref[-1])) > 1e-6
