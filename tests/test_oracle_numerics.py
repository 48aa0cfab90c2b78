"""Pins of the oracle's exact widening of stored values (CPU only).

Every bf16 parity comparison goes through ``oracle.bf16_bits_to_f64``.  These
tests tie it to values the 16-bit format itself fixes -- one sign bit, eight
exponent bits with bias 127, seven fraction bits, the top half of an IEEE
binary32 word -- written out here from the format's definition, not computed
by the function under test.  The 16-bit caches are the ones the pages price
("单请求 KV Cache", 显存代价: two bytes per value in bf16).
"""

import math

import numpy as np
import pytest

import oracle
from oracle.numerics import bf16_bits_to_f64, to_f64
from workloads import bf16_round_bits


def _widen(bits):
    return bf16_bits_to_f64(np.array([bits], dtype=np.uint16))[0]


# (bit pattern, value the format assigns to it)
FIXED = [
    (0x3F80, 1.0),                        # exponent 127, fraction 0
    (0xBF80, -1.0),
    (0x4000, 2.0),
    (0xC040, -3.0),                       # -(1 + 1/2) * 2^1
    (0x3F00, 0.5),
    (0x3FC0, 1.5),
    (0x3F81, 1.0 + 2.0 ** -7),            # one unit in the last place above 1
    (0x4049, 3.140625),                   # 1.5703125 * 2
    (0x0080, 2.0 ** -126),                # smallest normal
    (0x0001, 2.0 ** -133),                # smallest subnormal: 2^-126 * 2^-7
    (0x007F, 127 * 2.0 ** -133),          # largest subnormal
    (0x7F7F, (2 - 2.0 ** -7) * 2.0 ** 127),  # largest finite
    (0xFF7F, -(2 - 2.0 ** -7) * 2.0 ** 127),
    (0x0000, 0.0),
]


@pytest.mark.parametrize("bits,value", FIXED)
def test_fixed_patterns(bits, value):
    got = _widen(bits)
    assert got == value, (hex(bits), got, value)


def test_signed_zero_infinities_and_nan():
    nz = _widen(0x8000)
    assert nz == 0.0 and math.copysign(1.0, nz) == -1.0
    assert math.copysign(1.0, _widen(0x0000)) == 1.0
    assert _widen(0x7F80) == math.inf
    assert _widen(0xFF80) == -math.inf
    assert math.isnan(_widen(0x7FC0)) and math.isnan(_widen(0xFFC1))


@pytest.mark.filterwarnings("ignore:invalid value encountered in cast")
def test_every_pattern_against_the_format_definition():
    # All 65,536 patterns, decoded field by field from the definition.
    bits = np.arange(1 << 16, dtype=np.uint32)
    sign = np.where(bits >> 15, -1.0, 1.0)
    expo = ((bits >> 7) & 0xFF).astype(np.int64)
    frac = (bits & 0x7F).astype(np.float64)
    normal = sign * (1.0 + frac / 128.0) * np.ldexp(1.0, expo - 127)
    sub = sign * (frac / 128.0) * 2.0 ** -126
    want = np.where(expo == 0, sub, normal)
    got = bf16_bits_to_f64(bits.astype(np.uint16))
    finite = expo != 0xFF
    assert np.array_equal(got[finite], want[finite])
    # exponent all ones: infinities (fraction 0) and NaNs
    inf_mask = (expo == 0xFF) & (frac == 0)
    assert np.all(np.isinf(got[inf_mask]))
    assert np.all(np.isnan(got[(expo == 0xFF) & (frac != 0)]))
    # the sign bit survives on zeros
    assert np.array_equal(np.signbit(got[frac == 0]), (bits[frac == 0] >> 15).astype(bool))


def test_byte_order_is_the_value_not_the_memory():
    # A little-endian 0x3F80 is the bytes 80 3F; reading the bytes swapped
    # (0x803F) would give a tiny negative subnormal, not 1.
    raw = np.frombuffer(bytes([0x80, 0x3F]), dtype="<u2")
    assert bf16_bits_to_f64(raw)[0] == 1.0
    assert _widen(0x803F) == -(0x3F / 128.0) * 2.0 ** -126


def test_rejects_other_dtypes():
    for bad in (np.array([1.0], np.float32), np.array([0x3F80], np.int32),
                np.array([0x3F80], np.int16)):
        with pytest.raises(TypeError):
            bf16_bits_to_f64(bad)
    with pytest.raises(TypeError):
        to_f64(np.array([1.0], np.float64), "f32")
    with pytest.raises(TypeError):
        to_f64(np.array([1.0], np.float32), "bf16")
    with pytest.raises(ValueError):
        to_f64(np.array([1], np.uint16), "fp16")


def test_f32_widening_is_exact():
    x = np.array([1.0, -0.0, 2.0 ** -149, 3.4028234663852886e38, 0.1], np.float32)
    got = to_f64(x, "f32")
    assert got[0] == 1.0 and np.signbit(got[1]) and got[2] == 2.0 ** -149
    assert got[3] == (2 - 2.0 ** -23) * 2.0 ** 127
    assert got[4] == 13421773 * 2.0 ** -27  # the fp32 nearest to 0.1


def test_exact_bf16_values_round_trip_through_the_generator_rounding():
    # Values with at most 8 significant bits are bf16 numbers: rounding them
    # to bf16 and widening gives them back exactly.
    vals = np.array([1.0, -3.0, 0.5, 1.5, 1 + 2.0 ** -7, 2.0 ** -126, 2.0 ** -133, -0.0,
                     255.0 * 2.0 ** 100, 3.140625], dtype=np.float32)
    back = bf16_bits_to_f64(bf16_round_bits(vals))
    assert np.array_equal(back, vals.astype(np.float64))
    assert np.array_equal(np.signbit(back), np.signbit(vals))


def test_channel_scales_map_each_channel_max_to_the_largest_code():
    # Per-channel K scales of the FP8 cache ("KV-Cache——为什么AI回复越来越快",
    # KV-Cache量化: K scaled per channel): s = max|K| / 448 over the
    # calibration rows, so each channel's largest magnitude is the largest
    # finite E4M3 value, code 0x7E (0xFE when negative), and nothing saturates.
    rng = np.random.default_rng(31)
    K = (rng.standard_normal((300, 3, 16)) * rng.uniform(0.1, 10, (1, 3, 16))).astype(np.float32)
    ks = oracle.channel_scales_fp8(K)
    assert ks.shape == (3, 16) and ks.dtype == np.float32
    codes = oracle.quantize_fp8(K, ks)
    am = np.argmax(np.abs(K), axis=0)
    top = np.take_along_axis(codes, am[None], axis=0)[0]
    top_sign = np.take_along_axis(K, am[None], axis=0)[0] < 0
    assert np.all(top == np.where(top_sign, 0xFE, 0x7E))
    # no other code exceeds magnitude 0x7E, and 0x7F / 0xFF (NaN) never appear
    assert np.all((codes & 0x7F) <= 0x7E)
    # a row of three times the calibrated range saturates at 448
    big = oracle.quantize_fp8(np.float32(3) * np.abs(K).max(axis=0), ks)
    assert np.all(big == 0x7E)
    # a channel of zeros gets scale 0
    K[:, 1, 5] = 0
    assert oracle.channel_scales_fp8(K)[1, 5] == 0
