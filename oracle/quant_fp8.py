"""FP8 (E4M3) KV cache: per-channel K scales, per-token V scales (oracle).

Test infrastructure only.  Citation keys are listed in ``oracle/__init__.py``.

[DQ] "KV-Cache量化" quantises the FP16 K and V to FP8 (one byte), halving
the cache, with per-token scales for V and per-channel scales for K; [LC] 4
and [SW] list FP8/INT8 storage as orthogonal to paging.  The pages name FP8
but not its encoding.  Readings taken here:

* E4M3 as defined by the OCP 8-bit floating-point format (its "FN" form):
  sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 holds the
  subnormals m/8 * 2^-6; no infinities; S.1111.111 is NaN, so the largest
  finite magnitude is 1.75 * 2^8 = 448.
* code = E4M3(x / s): the correctly rounded fp32 quotient goes to the nearest
  E4M3 value, ties to the even code; magnitudes beyond 448 saturate to 448
  (a cache stores finite values).  The code's sign is the quotient's sign
  bit, so a negative quotient that rounds to zero is stored as -0 (0x80).
* Scales as for the INT8 cache, with 448 in place of 127: K per (K/V head,
  dimension) from a calibration (max |K| / 448), V per (token, K/V head)
  max |v| / 448 in fp32 when the row is appended (0 for an all-zero row).
* A stored value stands for E4M3(code) * s; attention over the cache is the
  plain decode attention applied to those values.
"""

import numpy as np

from .attention import decode_attention
from .numerics import to_f64
from .paged import _check_block, gather_logical, slot_of

E4M3_MAX = 448.0


def e4m3_value(code):
    """The number an E4M3 byte stands for (NaN for 0x7F and 0xFF)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_TABLE = np.array([e4m3_value(c) for c in range(256)])
# Non-negative finite codes 0x00 .. 0x7E in increasing value.
_POS = _TABLE[:0x7F]


def e4m3_decode(codes):
    """uint8 codes (any shape) -> fp64 values."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(y):
    """fp32 values -> E4M3 codes: nearest value, ties to the even code,
    saturation at 448, the sign bit of y kept."""
    y = np.asarray(y, dtype=np.float32)
    a = np.minimum(np.abs(y).astype(np.float64), E4M3_MAX)
    hi = np.searchsorted(_POS, a, side="left")          # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - _POS[lo], _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(y), mag | 0x80, mag).astype(np.uint8)


def quantize_fp8(x, s):
    """fp32 values and fp32 scales (broadcast) -> E4M3 codes of x / s."""
    x = np.asarray(x, dtype=np.float32)
    s = np.broadcast_to(np.asarray(s, dtype=np.float32), x.shape)
    q = np.zeros(x.shape, dtype=np.float32)
    nz = s > 0
    q[nz] = x[nz] / s[nz]  # fp32 / fp32: the correctly rounded quotient
    return e4m3_encode(q)


def channel_scales_fp8(K):
    """Per-channel K scales from a calibration set K [T, H_kv, d]."""
    K = np.asarray(K, dtype=np.float32)
    return (np.max(np.abs(K), axis=0) / np.float32(E4M3_MAX)).astype(np.float32)


def append_paged_fp8(kq_pool, vq_pool, vs_pool, k_new, v_new, dtype, k_scale, block_table,
                     seq_lens, block_size=16):
    """Quantise each sequence's new K/V row into its slot (E4M3 codes, V
    scale max |v| / 448); return new pools (uint8 codes, fp32 V scales)."""
    kq = np.array(kq_pool, copy=True)
    vq = np.array(vq_pool, copy=True)
    vs = np.array(vs_pool, copy=True)
    kf = to_f64(k_new, dtype).astype(np.float32)
    vf = to_f64(v_new, dtype).astype(np.float32)
    kc = quantize_fp8(kf, k_scale)
    vsc = (np.max(np.abs(vf), axis=-1) / np.float32(E4M3_MAX)).astype(np.float32)
    vc = quantize_fp8(vf, vsc[..., None])
    for b, length in enumerate(np.asarray(seq_lens)):
        if length < 1:
            raise ValueError("seq_lens must be >= 1 (the appended token is counted)")
        blk, off = slot_of(block_table, b, int(length) - 1, block_size)
        _check_block(blk, kq.shape[0])
        kq[blk, off] = kc[b]
        vq[blk, off] = vc[b]
        vs[blk, off] = vsc[b]
    return kq, vq, vs


def decode_attn_paged_fp8(q, kq_pool, vq_pool, vs_pool, k_scale, block_table, seq_lens, dtype,
                          scale=None, block_size=16):
    """Decode attention over an E4M3 paged cache holding every position
    [0, seq_lens[b]).  Returns fp64 [B, H_q, d]."""
    lens = np.asarray(seq_lens)
    ks = np.asarray(k_scale, dtype=np.float64)
    outs = []
    for b in range(lens.shape[0]):
        n = int(lens[b])
        K = e4m3_decode(gather_logical(kq_pool, block_table, b, n, block_size)) * ks
        V = (e4m3_decode(gather_logical(vq_pool, block_table, b, n, block_size)) *
             np.asarray(gather_logical(vs_pool, block_table, b, n, block_size),
                        dtype=np.float64)[..., None])
        outs.append(decode_attention(to_f64(q[b], dtype), K, V, scale))
    return np.stack(outs)
