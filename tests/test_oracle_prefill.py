"""Pins of the multi-row append and causal prefill oracle (CPU only).

Each row of a chunked prefill is checked against the decode formulation
(gather positions 0..p, plain attention) and one-row chunks against the
decode oracle with k_new / v_new; the many-slot append against repeated
single-row appends.
"""

import numpy as np

import oracle
from workloads import make_paged_prefill


def _inp(seed, past, new, H_q=4, H_kv=2, d=16):
    return make_paged_prefill(np.random.default_rng(seed), len(past), H_q, H_kv, d, past, new,
                              dtype="f32")


def _appended(inp):
    return oracle.append_paged_multi(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, inp.cu_rows,
                                     inp.block_table, inp.seq_lens)


def test_multi_append_equals_repeated_single_appends():
    inp = _inp(1, [0, 17, 40], [20, 5, 1])
    k2, v2 = _appended(inp)
    k1, v1 = inp.k_pool, inp.v_pool
    past = inp.seq_lens - np.diff(inp.cu_rows)
    for b in range(inp.B):
        for i in range(inp.cu_rows[b + 1] - inp.cu_rows[b]):
            lens = past.copy()
            lens[b] = past[b] + i + 1
            row = inp.cu_rows[b] + i
            kn = np.repeat(inp.k_new[row:row + 1], inp.B, axis=0)
            vn = np.repeat(inp.v_new[row:row + 1], inp.B, axis=0)
            sel = [b]
            k1, v1 = oracle.append_paged(k1, v1, kn[sel], vn[sel], inp.block_table[sel],
                                         lens[sel])
    assert np.array_equal(k1, k2, equal_nan=True) and np.array_equal(v1, v2, equal_nan=True)


def test_rows_equal_decode_over_their_prefix():
    inp = _inp(2, [0, 9, 33], [12, 7, 3], H_q=8, H_kv=2)
    k2, v2 = _appended(inp)
    out = oracle.prefill_attn_paged(inp.q, k2, v2, inp.block_table, inp.seq_lens, inp.cu_rows,
                                    "f32")
    for b in range(inp.B):
        n = inp.cu_rows[b + 1] - inp.cu_rows[b]
        L = int(inp.seq_lens[b])
        K = oracle.gather_logical(k2, inp.block_table, b, L).astype(np.float64)
        V = oracle.gather_logical(v2, inp.block_table, b, L).astype(np.float64)
        for i in range(n):
            p = L - n + i
            row = inp.cu_rows[b] + i
            want = oracle.decode_attention(inp.q[row].astype(np.float64), K[:p + 1], V[:p + 1])
            assert np.max(np.abs(out[row] - want)) < 1e-12


def test_first_prefill_row_is_its_own_value():
    inp = _inp(3, [0], [10])
    k2, v2 = _appended(inp)
    out = oracle.prefill_attn_paged(inp.q, k2, v2, inp.block_table, inp.seq_lens, inp.cu_rows,
                                    "f32")
    r = inp.H_q // inp.H_kv
    for h in range(inp.H_q):
        assert np.array_equal(out[0, h], inp.v_new[0, h // r].astype(np.float64))


def test_one_row_chunks_are_decode_steps():
    inp = _inp(4, [5, 100, 31], [1, 1, 1])
    k2, v2 = _appended(inp)
    got = oracle.prefill_attn_paged(inp.q, k2, v2, inp.block_table, inp.seq_lens, inp.cu_rows,
                                    "f32")
    want = oracle.decode_attn_paged(inp.q, inp.k_pool, inp.v_pool, inp.block_table,
                                    inp.seq_lens, "f32", inp.k_new, inp.v_new)
    assert np.max(np.abs(got - want)) < 1e-12
