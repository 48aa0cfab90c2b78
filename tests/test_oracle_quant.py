"""Pins of the INT8 cache oracle (CPU only).

The quantiser is checked against brute force (the nearest code among all
255), exact half steps, the clip bounds and the round-trip bound; the INT8
decode against the [SW] worked example and against plain attention on
inputs whose codes are exact, where applying a scale along the wrong axis
changes the result.
"""

import json
import os

import numpy as np
import pytest

import oracle
from oracle import quant


def test_half_steps_round_to_even_and_codes_clip():
    s = np.float32(0.25)  # a power of two: x / s is exact
    x = np.array([0.625, 0.875, -0.625, 0.125, 0.375, -0.375, 100.0, -100.0, 31.75],
                 dtype=np.float32)
    assert oracle.quantize(x, s).tolist() == [2, 4, -2, 0, 2, -2, 127, -127, 127]


def test_codes_are_the_nearest_of_all_codes():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((64, 4, 32)) * 3).astype(np.float32)
    codes, s = quant.quantize_v_rows(x)
    cand = np.arange(-127, 128, dtype=np.float64)
    xs = x.astype(np.float64) / s.astype(np.float64)[..., None]
    dist = np.abs(xs[..., None] - cand)
    best = dist.min(axis=-1)
    got = np.abs(xs - codes.astype(np.float64))
    # the chosen code is a nearest one (the fp32 quotient may differ from the
    # exact one by an ulp, which can only matter at a tie)
    assert np.all(got <= best + 1e-5)
    # each row's largest magnitude maps to +-127
    am = np.argmax(np.abs(x), axis=-1)
    top = np.take_along_axis(codes, am[..., None], axis=-1)[..., 0]
    assert np.all(np.abs(top) == 127)
    # round trip within half a step
    deq = quant.dequantize_v(codes, s)
    assert np.all(np.abs(deq - x) <= s.astype(np.float64)[..., None] * 0.5 * (1 + 1e-6))


def test_zero_row_has_zero_scale_and_codes():
    codes, s = quant.quantize_v_rows(np.zeros((1, 2, 8), dtype=np.float32))
    assert np.all(s == 0) and np.all(codes == 0)
    assert np.all(quant.dequantize_v(codes, s) == 0)


def test_channel_scales_cover_the_calibration_set():
    rng = np.random.default_rng(6)
    K = rng.standard_normal((200, 2, 16)).astype(np.float32)
    ks = oracle.channel_scales(K)
    assert ks.shape == (2, 16)
    codes = oracle.quantize(K, ks)
    assert np.all(np.abs(codes).max(axis=0) == 127)
    # a new row beyond the calibrated range clips
    assert oracle.quantize(np.float32(3) * K.max(axis=0), ks).max() == 127


def test_worked_example_through_the_int8_cache(golden_dir):
    # [SW] 知识点二: q = [0], V history [2], new V [4] -> [3]; one head, d = 1.
    ex = json.load(open(os.path.join(golden_dir, "worked_example.json")))["with_history"]
    table = np.array([[0]], dtype=np.int32)
    kq = np.zeros((1, 16, 1, 1), np.int8)
    vq = np.zeros((1, 16, 1, 1), np.int8)
    vs = np.zeros((1, 16, 1), np.float32)
    k_scale = np.full((1, 1), 2.0 / 127, np.float32)
    rows = [(ex["past_keys"][0], ex["past_values"][0]), (ex["new_key"], ex["new_value"])]
    for t, (k, v) in enumerate(rows):
        kq, vq, vs = oracle.append_paged_int8(
            kq, vq, vs, np.array([[k]], np.float32), np.array([[v]], np.float32), "f32",
            k_scale, table, [t + 1])
    q = np.array([[ex["query"]]], np.float32)
    out = oracle.decode_attn_paged_int8(q, kq, vq, vs, k_scale, table, [2], "f32")
    assert vq[0, :2, 0, 0].tolist() == [127, 127]
    assert out[0, 0].tolist() == pytest.approx(ex["output"], rel=1e-6)


def _exact_inputs(rng, T, H_kv, d):
    """K and V whose codes and power-of-two scales are exact: every channel
    of K and every token row of V reaches code +-127 once."""
    kc = rng.integers(-126, 127, size=(T, H_kv, d))
    kc[0] = 127
    ke = rng.integers(3, 9, size=(H_kv, d))
    vc = rng.integers(-126, 127, size=(T, H_kv, d))
    vc[..., 0] = -127
    ve = rng.integers(3, 9, size=(T, H_kv))
    K = (kc * 2.0 ** -ke).astype(np.float32)
    V = (vc * 2.0 ** -ve[..., None]).astype(np.float32)
    return K, V


def test_exact_codes_give_plain_attention_and_the_axes_matter():
    rng = np.random.default_rng(7)
    T, H_q, H_kv, d = 37, 4, 2, 16
    K, V = _exact_inputs(rng, T, H_kv, d)
    q = rng.standard_normal((H_q, d)).astype(np.float32)
    k_scale = oracle.channel_scales(K)
    nb = -(-T // 16)
    table = np.arange(nb, dtype=np.int32)[None, :]
    kq = np.zeros((nb, 16, H_kv, d), np.int8)
    vq = np.zeros((nb, 16, H_kv, d), np.int8)
    vs = np.zeros((nb, 16, H_kv), np.float32)
    for t in range(T):
        kq, vq, vs = oracle.append_paged_int8(kq, vq, vs, K[t:t + 1], V[t:t + 1], "f32",
                                              k_scale, table, [t + 1])
    got = oracle.decode_attn_paged_int8(q[None], kq, vq, vs, k_scale, table, [T], "f32")[0]
    want = oracle.decode_attention(q.astype(np.float64), K, V)
    assert np.max(np.abs(got - want)) < 1e-12
    # the codes reproduce the values exactly
    Kc = oracle.gather_logical(kq, table, 0, T)
    Vc = oracle.gather_logical(vq, table, 0, T)
    Vs = oracle.gather_logical(vs, table, 0, T)
    assert np.array_equal(oracle.dequantize_k(Kc, k_scale), K.astype(np.float64))
    assert np.array_equal(oracle.dequantize_v(Vc, Vs), V.astype(np.float64))
    # K's scale taken per token, or V's per channel, gives another answer
    wrong_k = Kc * Vs[..., None].astype(np.float64)
    wrong_v = Vc * k_scale.astype(np.float64)
    assert np.max(np.abs(oracle.decode_attention(q, wrong_k, V) - want)) > 1e-3
    assert np.max(np.abs(oracle.decode_attention(q, K, wrong_v) - want)) > 1e-3


def test_append_int8_writes_only_the_slots():
    rng = np.random.default_rng(8)
    B, H_kv, d, nb = 3, 2, 8, 6
    table = np.array([[4, 1], [0, 5], [2, 3]], dtype=np.int32)
    lens = [20, 5, 32]
    kq = rng.integers(-127, 128, size=(nb, 16, H_kv, d)).astype(np.int8)
    vq = rng.integers(-127, 128, size=(nb, 16, H_kv, d)).astype(np.int8)
    vs = rng.random((nb, 16, H_kv)).astype(np.float32)
    kn = rng.standard_normal((B, H_kv, d)).astype(np.float32)
    vn = rng.standard_normal((B, H_kv, d)).astype(np.float32)
    ks = np.full((H_kv, d), 0.02, np.float32)
    k2, v2, s2 = oracle.append_paged_int8(kq, vq, vs, kn, vn, "f32", ks, table, lens)
    slots = {oracle.slot_of(table, b, n - 1) for b, n in enumerate(lens)}
    for blk in range(nb):
        for off in range(16):
            same = (blk, off) not in slots
            assert np.array_equal(k2[blk, off], kq[blk, off]) == same
            assert np.array_equal(s2[blk, off], vs[blk, off]) == same
    blk, off = oracle.slot_of(table, 1, 4)
    assert np.array_equal(k2[blk, off], oracle.quantize(kn[1], ks))
    assert np.allclose(s2[blk, off], np.abs(vn[1]).max(axis=-1) / 127, rtol=1e-7)


def test_int8_halves_the_bytes_per_token():
    # [DQ] KV-Cache量化: one byte instead of two halves the cache.
    assert oracle.bytes_per_token(32, 8, 128, 1) * 2 == oracle.bytes_per_token(32, 8, 128, 2)
