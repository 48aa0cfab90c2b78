"""The parity check rejects plausible mistakes (planted in the oracle, on CPU).

Each case computes a deliberately wrong result with the oracle's own pieces
-- a zero output, an off-by-one length, the interleaved head grouping, a
K-only shuffle, a missing append -- and checks that the contract comparison
used by the GPU parity tests fails on it, at shapes like the workloads'.
"""

import numpy as np
import pytest

import oracle
from contract import contract_report
from workloads import make_paged_decode, make_mla


@pytest.fixture(scope="module")
def gqa():
    rng = np.random.default_rng(99)
    lens = [700, 1025, 1536, 2048 + 7]
    inp = make_paged_decode(rng, len(lens), 32, 8, 128, lens, dtype="bf16")
    ref = oracle.decode_attn_paged(inp.q, inp.k_pool, inp.v_pool, inp.block_table,
                                   inp.seq_lens, "bf16", inp.k_new, inp.v_new)
    return inp, ref


def _logical(inp, b):
    K = np.concatenate([oracle.to_f64(oracle.gather_history(inp.k_pool, inp.block_table,
                                                            inp.seq_lens, b), "bf16"),
                        oracle.to_f64(inp.k_new[b:b + 1], "bf16")])
    V = np.concatenate([oracle.to_f64(oracle.gather_history(inp.v_pool, inp.block_table,
                                                            inp.seq_lens, b), "bf16"),
                        oracle.to_f64(inp.v_new[b:b + 1], "bf16")])
    return oracle.to_f64(inp.q[b], "bf16"), K, V


def test_correct_result_passes(gqa):
    inp, ref = gqa
    noisy = ref * (1 + 1e-3 * np.random.default_rng(0).standard_normal(ref.shape))
    assert contract_report(noisy, ref)["ok"]


def test_zero_output_fails(gqa):
    _, ref = gqa
    assert not contract_report(np.zeros_like(ref), ref)["ok"]


def test_off_by_one_length_fails(gqa):
    inp, ref = gqa
    wrong = ref.copy()
    for b in range(inp.B):
        q, K, V = _logical(inp, b)
        wrong[b] = oracle.decode_attention(q, K[:-1], V[:-1])
    assert not contract_report(wrong, ref)["ok"]


def test_interleaved_grouping_fails(gqa):
    inp, ref = gqa
    wrong = ref.copy()
    for b in range(inp.B):
        q, K, V = _logical(inp, b)
        for h in range(inp.H_q):
            g = h % inp.H_kv  # interleaved instead of contiguous groups
            wrong[b, h] = oracle.decode_attention(q[h:h + 1], K[:, g:g + 1], V[:, g:g + 1])[0]
    assert not contract_report(wrong, ref)["ok"]


def test_key_only_shuffle_fails(gqa):
    inp, ref = gqa
    wrong = ref.copy()
    rng = np.random.default_rng(1)
    for b in range(inp.B):
        q, K, V = _logical(inp, b)
        wrong[b] = oracle.decode_attention(q, K[rng.permutation(K.shape[0])], V)
    assert not contract_report(wrong, ref)["ok"]


def test_missing_append_fails(gqa):
    inp, ref = gqa
    wrong = ref.copy()
    for b in range(inp.B):
        q, K, V = _logical(inp, b)
        K[-1] = 0.0
        V[-1] = 0.0
        wrong[b] = oracle.decode_attention(q, K, V)
    # a zeroed last row shifts the output a little; the scaled check must see it
    rep = contract_report(wrong, ref)
    assert not rep["ok"], rep


def test_mla_zero_output_fails_even_though_tiny():
    inp = make_mla(np.random.default_rng(5), 2, 16, 512, 64, [4096, 4000], std=1 / 24)
    ref = oracle.mla_decode_paged(inp.q, inp.c_pool, inp.block_table, inp.seq_lens, 512,
                                  1 / np.sqrt(192), c_new=inp.c_new)
    rep = contract_report(np.zeros_like(ref), ref)
    # the elementwise bound alone would accept zeros here
    assert rep["bound_ok"] and not rep["ok"]
