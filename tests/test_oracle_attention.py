"""Pins of the oracle's attention functions (CPU only).

Each test checks the oracle against something other than itself: values the
pages print, closed forms, invariants the pages state, special cases that
reduce to a simpler computation, and a second formulation (the full causal
score matrix) of the same mathematics.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# --- worked example and closed forms -------------------------------------

def _single_head(example):
    q = np.array([example["query"]])
    keys = [list(k) for k in example["past_keys"]] + [example["new_key"]]
    vals = [list(v) for v in example["past_values"]] + [example["new_value"]]
    K = np.array(keys)[:, None, :]
    V = np.array(vals)[:, None, :]
    return q, K, V


@pytest.mark.parametrize("case", ["with_history", "without_history"])
def test_worked_example(golden_dir, case):
    ex = json.load(open(os.path.join(golden_dir, "worked_example.json")))[case]
    q, K, V = _single_head(ex)
    out, w = oracle.decode_attention_weights(q, K, V)
    assert out[0].tolist() == ex["output"]
    assert w[0].tolist() == ex["weights"]


def test_closed_form_two_keys():
    # d = 1, q = [1], keys [1], [-1], values [2], [4]: scores 1 and -1, so the
    # first weight is 1/(1+e^-2) = (1 + tanh 1)/2 and o = 3 - tanh(1).
    q = np.array([[1.0]])
    K = np.array([[[1.0]], [[-1.0]]])
    V = np.array([[[2.0]], [[4.0]]])
    assert oracle.decode_attention(q, K, V)[0, 0] == pytest.approx(3 - math.tanh(1), abs=1e-15)
    # swapping only the keys changes the meaning: o = 3 + tanh(1)
    assert oracle.decode_attention(q, K[::-1], V)[0, 0] == pytest.approx(3 + math.tanh(1), abs=1e-15)
    # swapping the K/V pairs together leaves it unchanged
    assert oracle.decode_attention(q, K[::-1], V[::-1])[0, 0] == pytest.approx(3 - math.tanh(1), abs=1e-15)


def test_scale_is_inverse_sqrt_d():
    # d = 4, q = (1,1,1,1), keys (1,1,1,1) and 0: raw dots 4 and 0, scaled by
    # 1/sqrt(4) to 2 and 0; weights e^2/(e^2+1) and 1/(e^2+1).
    q = np.ones((1, 4))
    K = np.stack([np.ones((1, 4)), np.zeros((1, 4))])
    V = np.array([[[1.0]], [[0.0]]])
    expect = math.exp(2) / (math.exp(2) + 1)
    assert oracle.decode_attention(q, K, V)[0, 0] == pytest.approx(expect, abs=1e-15)


# --- invariants ------------------------------------------------------------

def test_joint_permutation_invariant_key_only_changes():
    rng = np.random.default_rng(0)
    T, H_q, H_kv, d = 37, 8, 2, 16
    q, K, V = _rand(rng, H_q, d), _rand(rng, T, H_kv, d), _rand(rng, T, H_kv, d)
    base = oracle.decode_attention(q, K, V)
    perm = rng.permutation(T)
    assert np.max(np.abs(oracle.decode_attention(q, K[perm], V[perm]) - base)) < 1e-14
    assert np.max(np.abs(oracle.decode_attention(q, K[perm], V) - base)) > 1e-3


def test_single_position_returns_its_value():
    rng = np.random.default_rng(1)
    q, K, V = _rand(rng, 4, 8), _rand(rng, 1, 2, 8), _rand(rng, 1, 2, 8)
    out = oracle.decode_attention(q, K, V)
    assert np.array_equal(out, np.repeat(V[0], 2, axis=0))


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(2)
    K, V = _rand(rng, 50, 1, 8), _rand(rng, 50, 1, 6)
    out = oracle.decode_attention(np.zeros((1, 8)), K, V)
    assert np.max(np.abs(out[0] - V[:, 0, :].mean(axis=0))) < 1e-14


def test_weights_sum_to_one():
    rng = np.random.default_rng(3)
    q, K, V = _rand(rng, 6, 16) * 5, _rand(rng, 300, 3, 16), _rand(rng, 300, 3, 16)
    _, w = oracle.decode_attention_weights(q, K, V)
    assert np.all(w >= 0)
    assert np.max(np.abs(w.sum(axis=1) - 1)) < 1e-14


def test_large_scores_do_not_overflow():
    # subtracting the maximum keeps exp finite for scores far beyond exp's range
    q = np.array([[1000.0]])
    K = np.array([[[1.0]], [[0.999]]])
    V = np.array([[[1.0]], [[-1.0]]])
    out = oracle.decode_attention(q, K, V)
    z = 1000.0 * 0.001  # score difference after scaling by 1/sqrt(1)
    assert out[0, 0] == pytest.approx(math.tanh(z / 2), abs=1e-12)


# --- cached decode equals the last row of full causal recompute -------------

def test_cached_decode_equals_full_recompute():
    # generation with a cache vs recomputing everything each step, in the
    # manner of the pages' numpy experiment: token embeddings projected by
    # fixed weights, one head of width 8.
    rng = np.random.default_rng(42)
    T, D, dk = 12, 64, 8
    x = _rand(rng, T, D)
    Wq, Wk, Wv = (_rand(rng, D, dk) * 0.02 for _ in range(3))
    Q, K, V = x @ Wq, x @ Wk, x @ Wv
    full = oracle.causal_attention(Q, K, V, past_len=0)
    for t in range(T):
        cached = oracle.decode_attention(Q[t:t + 1], K[:t + 1, None, :], V[:t + 1, None, :])
        assert np.max(np.abs(cached[0] - full[t])) < 1e-12
        last = oracle.causal_attention(Q[t:t + 1], K[:t + 1], V[:t + 1], past_len=t)
        assert np.max(np.abs(cached[0] - last[0])) < 1e-12


def test_causal_mask_pattern():
    # prefill (past_len 0): row i must not depend on keys/values j > i;
    # decode row (past_len 4, one query) sees all 5 positions.
    rng = np.random.default_rng(5)
    Q, K, V = _rand(rng, 4, 8), _rand(rng, 4, 8), _rand(rng, 4, 3)
    base = oracle.causal_attention(Q, K, V, past_len=0)
    for j in range(4):
        K2, V2 = K.copy(), V.copy()
        K2[j] += 10.0
        V2[j] += 10.0
        moved = oracle.causal_attention(Q, K2, V2, past_len=0)
        for i in range(4):
            changed = np.max(np.abs(moved[i] - base[i])) > 1e-9
            assert changed == (j <= i), (i, j)
    K5, V5 = _rand(rng, 5, 8), _rand(rng, 5, 3)
    row = oracle.causal_attention(Q[:1], K5, V5, past_len=4)
    for j in range(5):
        V6 = V5.copy()
        V6[j] += 1.0
        assert np.max(np.abs(oracle.causal_attention(Q[:1], K5, V6, past_len=4) - row)) > 1e-9


def test_tiny_config_multihead_recompute():
    # the tiny workload's shape: 4 heads, d_head 32, 129 positions
    rng = np.random.default_rng(7)
    T, H, d = 129, 4, 32
    q, K, V = _rand(rng, H, d), _rand(rng, T, H, d), _rand(rng, T, H, d)
    dec = oracle.decode_attention(q, K, V)
    for h in range(H):
        Qfull = np.concatenate([_rand(rng, T - 1, d), q[h:h + 1]])
        full = oracle.causal_attention(Qfull, K[:, h], V[:, h], past_len=0)
        assert np.max(np.abs(full[-1] - dec[h])) < 1e-12


# --- head grouping ----------------------------------------------------------

@pytest.mark.parametrize("H_q,H_kv", [(8, 2), (32, 8), (64, 8), (6, 1)])
def test_grouped_equals_repeated_heads(H_q, H_kv):
    rng = np.random.default_rng(H_q * 100 + H_kv)
    T, d = 40, 16
    q, K, V = _rand(rng, H_q, d), _rand(rng, T, H_kv, d), _rand(rng, T, H_kv, d)
    r = H_q // H_kv
    mha = oracle.decode_attention(q, np.repeat(K, r, axis=1), np.repeat(V, r, axis=1))
    assert np.max(np.abs(oracle.decode_attention(q, K, V) - mha)) < 1e-14
    # query head h uses K/V head h // r: head r-1 and head r read different groups
    if H_kv > 1:
        solo = oracle.decode_attention(q[r:r + 1], K[:, 1:2], V[:, 1:2])
        assert np.max(np.abs(solo[0] - mha[r])) < 1e-14


def test_brute_force_tiny_loops():
    # pure-Python loops over every head, position and component
    rng = np.random.default_rng(11)
    T, H, d = 9, 2, 4
    q, K, V = _rand(rng, H, d), _rand(rng, T, H, d), _rand(rng, T, H, d)
    out = oracle.decode_attention(q, K, V)
    for h in range(H):
        zs = [sum(q[h][j] * K[t][h][j] for j in range(d)) / math.sqrt(d) for t in range(T)]
        top = max(zs)
        es = [math.exp(z - top) for z in zs]
        tot = sum(es)
        for j in range(d):
            o = sum(es[t] * V[t][h][j] for t in range(T)) / tot
            assert abs(o - out[h][j]) < 1e-13


# --- split partitions and the log-sum-exp merge ------------------------------

@pytest.mark.parametrize("partition", [1, 16, 100, 512, 10_000])
def test_split_merge_equals_direct(partition):
    rng = np.random.default_rng(partition)
    T, H_q, H_kv, d = 1000, 8, 2, 16
    q, K, V = _rand(rng, H_q, d) * 3, _rand(rng, T, H_kv, d), _rand(rng, T, H_kv, d)
    direct = oracle.decode_attention(q, K, V)
    split = oracle.decode_attention_split(q, K, V, partition)
    assert np.max(np.abs(split - direct)) < 1e-13


def test_merge_ignores_empty_partitions():
    rng = np.random.default_rng(9)
    q, K, V = _rand(rng, 8), _rand(rng, 30, 8), _rand(rng, 30, 4)
    parts = oracle.split_partials(q, K, V, 0.3, 16)
    with_empty = parts + [(-math.inf, 0.0, np.zeros(4))]
    assert np.array_equal(oracle.lse_merge(with_empty), oracle.lse_merge(parts))
    with pytest.raises(ValueError):
        oracle.lse_merge([(-math.inf, 0.0, np.zeros(4))])


# --- absorbed MLA -------------------------------------------------------------

def test_mla_is_mqa_with_latent_values():
    rng = np.random.default_rng(13)
    H, T, d_c, d_r = 16, 70, 512, 64
    q, C = _rand(rng, H, d_c + d_r) / 24, _rand(rng, T, d_c + d_r) / 24
    scale = 1 / math.sqrt(192)
    mla = oracle.mla_decode(q, C, d_c, scale)
    mqa = oracle.decode_attention(q, C[:, None, :], C[:, None, :d_c], scale=scale)
    assert np.max(np.abs(mla - mqa)) < 1e-15


def test_mla_absorption_identity():
    # Explicit per-head attention with k = [W_UK c ; k_R], v = W_UV c and
    # q = [q_C ; q_R] equals W_UV applied to the absorbed latent-space output
    # with q~_c = W_UK^T q_C.
    rng = np.random.default_rng(17)
    H, d_h, d_r, T = 3, 4, 2, 11
    d_c = 4 * d_h
    W_uk, W_uv = _rand(rng, H, d_h, d_c), _rand(rng, H, d_h, d_c)
    c, k_r = _rand(rng, T, d_c), _rand(rng, T, d_r)
    q_c, q_r = _rand(rng, H, d_h), _rand(rng, H, d_r)
    scale = 1 / math.sqrt(d_h + d_r)
    rows = np.concatenate([c, k_r], axis=1)
    for h in range(H):
        k = np.concatenate([c @ W_uk[h].T, k_r], axis=1)        # [T, d_h + d_r]
        v = c @ W_uv[h].T                                       # [T, d_h]
        qh = np.concatenate([q_c[h], q_r[h]])[None, :]
        explicit = oracle.decode_attention(qh, k[:, None, :], v[:, None, :], scale=scale)[0]
        q_tilde = np.concatenate([W_uk[h].T @ q_c[h], q_r[h]])[None, :]
        latent = oracle.mla_decode(q_tilde, rows, d_c, scale)[0]
        assert np.max(np.abs(W_uv[h] @ latent - explicit)) < 1e-13


# --- validation, as in the pages' cached-attention sketch -------------------------

def test_rejects_bad_inputs():
    q = np.zeros((2, 4))
    with pytest.raises(ValueError):
        oracle.decode_attention(q, np.zeros((0, 1, 4)), np.zeros((0, 1, 4)))
    with pytest.raises(ValueError):
        oracle.decode_attention(q, np.zeros((3, 1, 5)), np.zeros((3, 1, 4)))
    with pytest.raises(ValueError):
        oracle.decode_attention(np.zeros((3, 4)), np.zeros((3, 2, 4)), np.zeros((3, 2, 4)))
    K = np.zeros((3, 1, 4))
    K[1, 0, 2] = np.nan
    with pytest.raises(ValueError):
        oracle.decode_attention(q, K, np.zeros((3, 1, 4)))
