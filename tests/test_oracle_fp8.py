"""Pins of the FP8 (E4M3) cache oracle (CPU only).

The decoder is checked against values the E4M3 definition fixes (the OCP
8-bit format: bias 7, 3 mantissa bits, subnormals, 448 largest, S.1111.111
NaN), the encoder against exact ties, saturation, signed zero, brute force
over all 254 finite codes and the round trip; the FP8 decode against the
[SW] 知识点二 worked example and against plain attention on inputs whose
codes are exact, where a scale applied along the wrong axis changes the
result.
"""

import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x30, 0.5), (0x38, 1.0), (0x39, 1.125), (0x3F, 1.875), (0x40, 2.0), (0x7E, 448.0),
    (0x7D, 416.0), (0xB8, -1.0), (0xC0, -2.0), (0xFE, -448.0), (0x81, -(2.0 ** -9)),
])
def test_decode_fixed_values(code, value):
    assert oracle.e4m3_value(code) == value


def test_decode_specials():
    assert np.isnan(oracle.e4m3_value(0x7F)) and np.isnan(oracle.e4m3_value(0xFF))
    z = oracle.e4m3_value(0x80)
    assert z == 0.0 and np.signbit(z)
    # 126 distinct positive finite values, strictly increasing with the code
    v = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)
    # the step is 2^(e - 10) inside a binade and 2^-9 among the subnormals
    assert v[9] - v[8] == 2.0 ** -9 and v[0x39] - v[0x38] == 0.125


@pytest.mark.parametrize("y,code", [
    (1.0625, 0x38),        # halfway 1.0 .. 1.125: even code 0x38
    (1.1875, 0x3A),        # halfway 1.125 .. 1.25: even code 0x3A
    (2.0 ** -10, 0x00),    # half the smallest subnormal: to zero
    (3 * 2.0 ** -10, 0x02),  # halfway 2^-9 .. 2^-8
    (5 * 2.0 ** -10, 0x02),  # halfway 2^-8 .. 3 * 2^-9
    (15 * 2.0 ** -10, 0x08),  # halfway 7 * 2^-9 .. 2^-6 (subnormal to normal)
    (432.0, 0x7E),         # halfway 416 .. 448: even code 0x7E
    (449.0, 0x7E), (460.0, 0x7E), (1e9, 0x7E), (-1e9, 0xFE),
    (-2.0 ** -11, 0x80),   # a negative quotient that rounds to zero keeps its sign
    (0.0, 0x00),
])
def test_encode_ties_saturation_and_sign(y, code):
    assert int(oracle.e4m3_encode(np.float32(y))) == code


def test_encode_is_the_nearest_code_by_brute_force():
    rng = np.random.default_rng(8)
    y = np.concatenate([rng.standard_normal(4000) * 10, rng.standard_normal(2000) * 1e-3,
                        rng.uniform(-500, 500, 2000)]).astype(np.float32)
    codes = oracle.e4m3_encode(y)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.e4m3_decode(finite)
    yc = np.clip(y.astype(np.float64), -448.0, 448.0)
    best = np.min(np.abs(yc[:, None] - vals[None, :]), axis=1)
    got = np.abs(yc - oracle.e4m3_decode(codes))
    assert np.all(got == best)


def test_round_trip_of_every_finite_code():
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        v = np.float32(oracle.e4m3_value(c))
        back = int(oracle.e4m3_encode(np.float32(-0.0) if c == 0x80 else v))
        assert back == c, hex(c)


def test_scales_and_append_round_trip():
    rng = np.random.default_rng(9)
    v = (rng.standard_normal((3, 2, 16)) * 4).astype(np.float32)
    nb = 3
    kq = np.zeros((nb, 16, 2, 16), np.uint8)
    vq = np.zeros_like(kq)
    vs = np.zeros((nb, 16, 2), np.float32)
    table = np.array([[2], [0], [1]], np.int32)
    lens = np.array([5, 16, 1], np.int32)
    ks = oracle.channel_scales_fp8(v)
    kq2, vq2, vs2 = oracle.append_paged_fp8(kq, vq, vs, v, v, "f32", ks, table, lens)
    for b, (blk, off) in enumerate([(2, 4), (0, 15), (1, 0)]):
        # each row's largest magnitude maps to +-448 exactly
        am = np.argmax(np.abs(v[b]), axis=-1)
        top = np.take_along_axis(vq2[blk, off], am[:, None], axis=-1)[:, 0]
        assert np.all(oracle.e4m3_decode(top & 0x7F) == 448.0)
        # dequantised values within half a step of 3 mantissa bits (relative 1/16)
        deq = oracle.e4m3_decode(vq2[blk, off]) * vs2[blk, off][:, None]
        err = np.abs(deq - v[b])
        assert np.all(err <= np.abs(v[b]) / 16 + vs2[blk, off][:, None] * 2.0 ** -10)
    # untouched slots stay zero
    mask = np.ones(kq.shape[:2], bool)
    mask[2, 4] = mask[0, 15] = mask[1, 0] = False
    assert np.all(kq2[mask] == 0) and np.all(vq2[mask] == 0)


def test_decode_worked_example_and_scale_axes():
    # [SW] 知识点二: q = [0], history V = [2], new V = [4] -> 3.  With codes
    # exact (2 = 0x40, 4 = 0x48) and unit scales the FP8 path gives 3.
    kq = np.zeros((1, 16, 1, 1), np.uint8)
    vq = np.zeros_like(kq)
    vq[0, 0, 0, 0], vq[0, 1, 0, 0] = 0x40, 0x48
    vs = np.ones((1, 16, 1), np.float32)
    q = np.zeros((1, 1, 1), np.float32)
    out = oracle.decode_attn_paged_fp8(q, kq, vq, vs, np.ones((1, 1), np.float32),
                                       np.array([[0]], np.int32), [2], "f32")
    assert out[0, 0, 0] == 3.0
    # per-channel K scales and per-token V scales: plain attention on the
    # dequantised rows; swapping the axes of the scales changes the output
    rng = np.random.default_rng(10)
    T, d = 16, 4
    kq = rng.integers(0, 0x7E, size=(1, 16, 1, d)).astype(np.uint8)
    vq = rng.integers(0, 0x7E, size=(1, 16, 1, d)).astype(np.uint8)
    ks = np.array([[0.5, 1.0, 2.0, 0.25]], np.float32)
    vs = rng.uniform(0.5, 2, size=(1, 16, 1)).astype(np.float32)
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    got = oracle.decode_attn_paged_fp8(q, kq, vq, vs, ks, np.array([[0]], np.int32), [T], "f32")
    K = oracle.e4m3_decode(kq[0, :, 0]) * ks[0].astype(np.float64)
    V = oracle.e4m3_decode(vq[0, :, 0]) * vs[0, :, 0].astype(np.float64)[:, None]
    ref = oracle.decode_attention(q[0].astype(np.float64), K[:, None, :], V[:, None, :])
    assert np.allclose(got, ref, rtol=0, atol=1e-14)
    Kw = oracle.e4m3_decode(kq[0, :, 0]) * vs[0, :, 0].astype(np.float64)[:, None]
    wrong = oracle.decode_attention(q[0].astype(np.float64), Kw[:, None, :], V[:, None, :])
    assert not np.allclose(got, wrong, atol=1e-6)
