"""INT8 KV cache: per-channel K scales, per-token V scales (oracle).

Test infrastructure only.  Citation keys are listed in ``oracle/__init__.py``.

[DQ] "KV-Cache量化" stores K and V in one byte instead of two, which halves
the cache and the bytes a decode step reads.  It names the granularities:
K is scaled per channel (every dimension of an attention head has its own
scale, since K's distribution changes little from token to token) and V per
token (every token's row has its own scale, since V varies more); the usual
choice it reports is INT8 for both.  [LC] 4 and [SW] list the same FP8/INT8
storage as orthogonal to paging and head sharing.

The page gives the granularity, not the arithmetic.  Readings taken here:

* Symmetric codes in [-127, 127]: code = clip(round(x / s), -127, 127), with
  round-half-to-even, and the stored value stands for code * s.
* K scales: one fp32 per (K/V head, dimension), an input of the caller (a
  calibration over the history; the seeded workloads take max |K| / 127 per
  channel).  Values of a new token beyond the calibrated range clip.
* V scale: one fp32 per (token, K/V head), s = max_j |v_j| / 127 when the row
  is appended (s = 0 and all codes 0 for an all-zero row), kept beside the
  cache in a pool [num_blocks, 16, H_kv] addressed like the rows.
* The decision that yields a code is taken in fp32: x and s are fp32 values,
  x / s is the correctly rounded fp32 quotient and max |v| / 127 the correctly
  rounded fp32 scale.  Dequantised values code * s are exact in fp64.
* Attention over the INT8 cache is the plain decode attention of
  ``attention.decode_attention`` applied to the dequantised K and V.
"""

import numpy as np

from .attention import decode_attention
from .numerics import to_f64
from .paged import _check_block, gather_history, gather_logical, slot_of

CODE_MAX = 127


def quantize(x, s):
    """fp32 values ``x`` and fp32 scales ``s`` (broadcast) -> int8 codes."""
    x = np.asarray(x, dtype=np.float32)
    s = np.broadcast_to(np.asarray(s, dtype=np.float32), x.shape)
    q = np.zeros(x.shape, dtype=np.float32)
    nz = s > 0
    q[nz] = x[nz] / s[nz]  # fp32 / fp32: the correctly rounded quotient
    q = np.clip(np.rint(q), -CODE_MAX, CODE_MAX)  # rint: half to even
    return q.astype(np.int8)


def channel_scales(K):
    """Per-channel K scales from a calibration set K [T, H_kv, d]: max over
    the tokens of |K| / 127 per (head, dimension), fp32."""
    K = np.asarray(K, dtype=np.float32)
    return (np.max(np.abs(K), axis=0) / np.float32(CODE_MAX)).astype(np.float32)


def _stored_f32(x, dtype):
    """Stored bf16 bits or fp32 values -> fp32 (exact)."""
    return to_f64(x, dtype).astype(np.float32)


def quantize_k_rows(k, k_scale):
    """K rows [..., H_kv, d] (fp32) -> codes with the per-channel scales."""
    return quantize(k, k_scale)


def quantize_v_rows(v):
    """V rows [..., H_kv, d] (fp32) -> (codes, scales [..., H_kv])."""
    v = np.asarray(v, dtype=np.float32)
    s = (np.max(np.abs(v), axis=-1) / np.float32(CODE_MAX)).astype(np.float32)
    return quantize(v, s[..., None]), s


def append_paged_int8(kq_pool, vq_pool, vs_pool, k_new, v_new, dtype, k_scale, block_table,
                      seq_lens, block_size=16):
    """Quantise each sequence's new K/V row into its slot; return new pools.

    k_new, v_new: stored values [B, H_kv, d] in ``dtype`` ('bf16' bits or
    'f32'); k_scale: fp32 [H_kv, d].  The slot is the one of
    ``paged.append_paged`` (position seq_lens[b] - 1 through the block
    table); the codes go to kq_pool / vq_pool [NB, 16, H_kv, d] (int8) and
    the V scales to vs_pool [NB, 16, H_kv] (fp32).  Copies are returned.
    """
    kq = np.array(kq_pool, copy=True)
    vq = np.array(vq_pool, copy=True)
    vs = np.array(vs_pool, copy=True)
    kf = _stored_f32(k_new, dtype)
    vf = _stored_f32(v_new, dtype)
    kc = quantize_k_rows(kf, k_scale)
    vc, vsc = quantize_v_rows(vf)
    for b, length in enumerate(np.asarray(seq_lens)):
        if length < 1:
            raise ValueError("seq_lens must be >= 1 (the appended token is counted)")
        blk, off = slot_of(block_table, b, int(length) - 1, block_size)
        _check_block(blk, kq.shape[0])
        kq[blk, off] = kc[b]
        vq[blk, off] = vc[b]
        vs[blk, off] = vsc[b]
    return kq, vq, vs


def dequantize_k(codes, k_scale):
    """K codes [T, H_kv, d] -> fp64 values code * scale[h, j]."""
    return np.asarray(codes, dtype=np.float64) * np.asarray(k_scale, dtype=np.float64)


def dequantize_v(codes, v_scale):
    """V codes [T, H_kv, d] and token scales [T, H_kv] -> fp64 values."""
    return np.asarray(codes, dtype=np.float64) * np.asarray(v_scale, dtype=np.float64)[..., None]


def decode_attn_paged_int8(q, kq_pool, vq_pool, vs_pool, k_scale, block_table, seq_lens, dtype,
                           scale=None, block_size=16):
    """Decode attention over an INT8 paged cache that already holds every
    position [0, seq_lens[b]) (history and this step's row).

    q: stored values [B, H_q, d] in ``dtype``.  Returns fp64 [B, H_q, d].
    """
    lens = np.asarray(seq_lens)
    outs = []
    for b in range(lens.shape[0]):
        n = int(lens[b])
        K = dequantize_k(gather_logical(kq_pool, block_table, b, n, block_size), k_scale)
        V = dequantize_v(gather_logical(vq_pool, block_table, b, n, block_size),
                         gather_logical(vs_pool, block_table, b, n, block_size))
        outs.append(decode_attention(to_f64(q[b], dtype), K, V, scale))
    return np.stack(outs)

