"""Single-query decode attention in fp64 (oracle; test infrastructure only).

Citation keys are listed in ``oracle/__init__.py``.  Decode attention is
exact attention, not an approximation, so the oracle is the plain definition:

  z_i = scale * q . k_i          (scale = 1/sqrt(d) unless given)
  a_i = exp(z_i - max z) / sum_j exp(z_j - max z)
  o   = sum_i a_i v_i

([SW] 知识点二, the z / a / o equations; [DQ] 02 "Self-Attention回顾", the
scaled dot-product attention formula; [DQ] 05 ``attention``: the stable
softmax subtracts the row maximum).  A decode step has a single query row,
which sees every cached position including its own ([MV] 改动三, the decode
mask row is all-visible).

Head grouping ([DQ] 03 "三种Attention架构"; [LC] 2.2 "路线一：架构压缩"):
H_q query heads share H_kv K/V heads, r = H_q / H_kv query heads per group.
The pages do not say which query heads form a group; the reading taken here
is contiguous groups, query head h reads K/V head h // r.

Split-KV partials and their log-sum-exp merge are not on the pages; they are
the exact algebraic regrouping of the same sums (see ``split_partials``).

Absorbed MLA ([LC] 2.2, the MLA equations and the note that W^UK / W^UV are
absorbed into the query / output projections; [LC] 4 "MLA 的工程含义"): the
cache holds one row per token, the latent c_t (d_c) concatenated with the
decoupled RoPE key (d_R).  With the absorbed query q~ = [q~_c ; q_R] the
scores are scale * q~ . row_t and the output, in latent space, is
sum_t a_t c_t.
"""

import math

import numpy as np

from .numerics import to_f64
from .paged import gather_history, gather_logical


def _check_finite(*arrays):
    for a in arrays:
        if not np.all(np.isfinite(a)):
            raise ValueError("inputs must be finite")


def decode_attention_weights(q, K, V, scale=None):
    """Decode attention for one sequence; returns (output, weights).

    q: [H_q, d]; K: [T, H_kv, d]; V: [T, H_kv, dv]  (any real dtype; fp64 used)
    Returns o [H_q, dv] and the normalised weights a [H_q, T].
    Rejects empty K/V, mismatched widths, H_q not a multiple of H_kv and
    non-finite values, as the cached-attention sketch of [SW] 知识点二 does.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if q.ndim != 2 or K.ndim != 3 or V.ndim != 3:
        raise ValueError("expected q [H_q, d], K [T, H_kv, d], V [T, H_kv, dv]")
    T, H_kv, d = K.shape
    H_q = q.shape[0]
    if T < 1 or d < 1 or V.shape[2] < 1:
        raise ValueError("K/V must be non-empty")
    if V.shape[0] != T or V.shape[1] != H_kv or q.shape[1] != d:
        raise ValueError("q, K and V shapes disagree")
    if H_kv < 1 or H_q % H_kv != 0:
        raise ValueError("H_q must be a positive multiple of H_kv")
    _check_finite(q, K, V)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    r = H_q // H_kv
    out = np.empty((H_q, V.shape[2]), dtype=np.float64)
    weights = np.empty((H_q, T), dtype=np.float64)
    for h in range(H_q):
        g = h // r
        z = scale * (K[:, g, :] @ q[h])
        e = np.exp(z - z.max())
        a = e / e.sum()
        weights[h] = a
        out[h] = a @ V[:, g, :]
    return out, weights


def decode_attention(q, K, V, scale=None):
    """Output only of :func:`decode_attention_weights`."""
    return decode_attention_weights(q, K, V, scale)[0]


def decode_attn_paged(q, k_pool, v_pool, block_table, seq_lens, dtype,
                      k_new=None, v_new=None, scale=None, block_size=16):
    """Decode attention for a batch whose K/V live in a paged pool.

    q: [B, H_q, d] stored values; pools: [NB, block_size, H_kv, d] stored
    values; ``dtype`` names the storage ('bf16' bit patterns or 'f32').
    If ``k_new``/``v_new`` ([B, H_kv, d]) are given, the pools hold only the
    history (positions < seq_lens[b] - 1) and the new row is appended
    logically, exactly as [SW] 知识点二 appends the current K/V to the history
    before attending; otherwise the pools already hold all seq_lens[b] rows.
    Returns fp64 [B, H_q, dv].
    """
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new or neither")
    lens = np.asarray(seq_lens)
    B = lens.shape[0]
    outs = []
    for b in range(B):
        if k_new is not None:
            K = np.concatenate([
                to_f64(gather_history(k_pool, block_table, lens, b, block_size), dtype),
                to_f64(np.asarray(k_new)[b:b + 1], dtype)])
            V = np.concatenate([
                to_f64(gather_history(v_pool, block_table, lens, b, block_size), dtype),
                to_f64(np.asarray(v_new)[b:b + 1], dtype)])
        else:
            K = to_f64(gather_logical(k_pool, block_table, b, lens[b], block_size), dtype)
            V = to_f64(gather_logical(v_pool, block_table, b, lens[b], block_size), dtype)
        outs.append(decode_attention(to_f64(np.asarray(q)[b], dtype), K, V, scale))
    return np.stack(outs)


def window_start(length, window):
    """First visible position of a decode row at position length - 1 under a
    sliding window of ``window`` positions.

    [DQ] "Window Attention / Sliding Window": only the most recent W tokens'
    K/V are kept and attended to; [SW] (the note after the worked example):
    the states outside the window may be dropped because the model's visible
    range itself is different.  Reading taken: the W most recent positions
    include the current one, so the row sees [max(0, length - W), length).
    """
    if window < 1:
        raise ValueError("window must be >= 1")
    return max(0, int(length) - int(window))


def decode_attn_paged_window(q, k_pool, v_pool, block_table, seq_lens, dtype, window,
                             k_new=None, v_new=None, scale=None, block_size=16):
    """``decode_attn_paged`` restricted to the sliding window: sequence b
    attends to positions [window_start(seq_lens[b], window), seq_lens[b]).
    With k_new / v_new the pools hold the history and the new row is the last
    position, as in ``decode_attn_paged``.  Returns fp64 [B, H_q, dv]."""
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new or neither")
    lens = np.asarray(seq_lens)
    outs = []
    for b in range(lens.shape[0]):
        n = int(lens[b])
        start = window_start(n, window)
        if k_new is not None:
            K = np.concatenate([
                to_f64(gather_history(k_pool, block_table, lens, b, block_size), dtype),
                to_f64(np.asarray(k_new)[b:b + 1], dtype)])
            V = np.concatenate([
                to_f64(gather_history(v_pool, block_table, lens, b, block_size), dtype),
                to_f64(np.asarray(v_new)[b:b + 1], dtype)])
        else:
            K = to_f64(gather_logical(k_pool, block_table, b, n, block_size), dtype)
            V = to_f64(gather_logical(v_pool, block_table, b, n, block_size), dtype)
        outs.append(decode_attention(to_f64(np.asarray(q)[b], dtype), K[start:], V[start:], scale))
    return np.stack(outs)


def split_partials(q_h, K_g, V_g, scale, partition):
    """Per-partition (m_p, l_p, o_p) of one query head over its K/V head.

    The positions [0, T) are cut into consecutive chunks of ``partition``
    tokens.  For chunk p with scores z_i:  m_p = max z,  l_p = sum e^{z_i - m_p},
    o_p = sum e^{z_i - m_p} v_i / l_p.  These are the stable-softmax pieces of
    the definition restricted to the chunk.
    q_h: [d]; K_g: [T, d]; V_g: [T, dv].
    """
    q_h = np.asarray(q_h, dtype=np.float64)
    K_g = np.asarray(K_g, dtype=np.float64)
    V_g = np.asarray(V_g, dtype=np.float64)
    if partition < 1:
        raise ValueError("partition must be >= 1")
    T = K_g.shape[0]
    if T < 1:
        raise ValueError("K/V must be non-empty")
    parts = []
    for start in range(0, T, partition):
        stop = min(start + partition, T)
        z = scale * (K_g[start:stop] @ q_h)
        m = z.max()
        e = np.exp(z - m)
        l = e.sum()
        parts.append((m, l, (e @ V_g[start:stop]) / l))
    return parts


def lse_merge(parts):
    """Merge partition partials into the full-softmax output.

    With M = max_p m_p, the full numerator is sum_p e^{m_p - M} l_p o_p and
    the full denominator sum_p e^{m_p - M} l_p; their ratio is the output.
    Empty partitions (l_p = 0, m_p = -inf) contribute nothing.
    """
    live = [(m, l, o) for (m, l, o) in parts if l > 0]
    if not live:
        raise ValueError("no non-empty partition to merge")
    M = max(m for m, _, _ in live)
    num = sum(math.exp(m - M) * l * o for m, l, o in live)
    den = sum(math.exp(m - M) * l for m, l, _ in live)
    return num / den


def decode_attention_split(q, K, V, partition, scale=None):
    """Decode attention computed per partition and merged by log-sum-exp.

    Same arguments as :func:`decode_attention` plus ``partition`` (tokens).
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    H_q, d = q.shape
    H_kv = K.shape[1]
    if H_q % H_kv != 0:
        raise ValueError("H_q must be a multiple of H_kv")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    r = H_q // H_kv
    out = np.empty((H_q, V.shape[2]), dtype=np.float64)
    for h in range(H_q):
        g = h // r
        out[h] = lse_merge(split_partials(q[h], K[:, g, :], V[:, g, :], scale, partition))
    return out


def mla_decode(q, C, d_c, scale):
    """Absorbed-MLA decode for one sequence, output in latent space.

    q: [H, d_c + d_R] absorbed queries [q~_c ; q_R]; C: [T, d_c + d_R] cached
    rows [c_t ; k^R_t] (latent first, then the decoupled RoPE key).
    z_t = scale * q . C_t over the full row; o = sum_t softmax(z)_t C_t[:d_c].
    Returns [H, d_c] in fp64.
    """
    q = np.asarray(q, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    if C.ndim != 2 or q.ndim != 2 or q.shape[1] != C.shape[1]:
        raise ValueError("expected q [H, w] and C [T, w] of the same width")
    if C.shape[0] < 1 or not (0 < d_c <= C.shape[1]):
        raise ValueError("empty cache or bad latent width")
    _check_finite(q, C)
    out = np.empty((q.shape[0], d_c), dtype=np.float64)
    for h in range(q.shape[0]):
        z = scale * (C @ q[h])
        e = np.exp(z - z.max())
        out[h] = (e @ C[:, :d_c]) / e.sum()
    return out


def mla_decode_paged(q, c_pool, block_table, seq_lens, d_c, scale, dtype="bf16",
                     c_new=None, block_size=16):
    """Absorbed-MLA decode over a paged latent pool [NB, block_size, w].

    If ``c_new`` ([B, w]) is given, the pool holds only the history and the
    new row is appended logically; otherwise the pool holds all rows.
    Returns fp64 [B, H, d_c].
    """
    lens = np.asarray(seq_lens)
    outs = []
    for b in range(lens.shape[0]):
        if c_new is not None:
            C = np.concatenate([
                to_f64(gather_history(c_pool, block_table, lens, b, block_size), dtype),
                to_f64(np.asarray(c_new)[b:b + 1], dtype)])
        else:
            C = to_f64(gather_logical(c_pool, block_table, b, lens[b], block_size), dtype)
        outs.append(mla_decode(to_f64(np.asarray(q)[b], dtype), C, d_c, scale))
    return np.stack(outs)


def causal_attention(Q, K, V, past_len, scale=None, window=None):
    """Full causal attention of n new rows over past_len cached + n new rows.

    Q: [n, d]; K: [past_len + n, d]; V: [past_len + n, dv].  Query row i sees
    key j exactly when j <= past_len + i ([MV] 改动三: ``mask[i, :past_len+i+1]``
    is visible; with past_len = 0 this is the lower-triangular prefill mask,
    with n = 1 the all-visible decode row).  With ``window`` W, row i also
    needs j > past_len + i - W (the band of the W most recent positions, [DQ]
    "Window Attention / Sliding Window").  The whole score matrix is formed,
    masked with -inf and normalised row by row.  Returns [n, dv].
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    n, d = Q.shape
    total = K.shape[0]
    if total != past_len + n or V.shape[0] != total:
        raise ValueError("K/V must hold past_len + n rows")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    scores = scale * (Q @ K.T)
    visible = np.arange(total)[None, :] <= (past_len + np.arange(n))[:, None]
    if window is not None:
        visible &= np.arange(total)[None, :] > (past_len + np.arange(n))[:, None] - window
    scores = np.where(visible, scores, -np.inf)
    scores = scores - scores.max(axis=1, keepdims=True)
    p = np.exp(scores)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ V


def prefill_attn_paged(q_rows, k_pool, v_pool, block_table, seq_lens, cu_rows, dtype,
                       scale=None, block_size=16):
    """Causal attention of n_b new rows per sequence over a paged cache that
    already holds every position [0, seq_lens[b]) (history and the new rows).

    Row i of sequence b sits at position p = seq_lens[b] - n_b + i and sees
    positions 0..p ([MV] 改动三: mask[i, :past_len + i + 1] is visible; with
    past_len = 0 the lower triangle of prefill, with n_b = 1 the decode row;
    [SW] 知识点二: each new query attends to the cache plus the new rows before
    it).  q_rows: [N, H_q, d] stored values in row order of cu_rows; returns
    fp64 [N, H_q, d].  Heads share K/V in contiguous groups as in
    ``decode_attention``.
    """
    cu = np.asarray(cu_rows)
    q_rows = np.asarray(q_rows)
    N, H_q, _ = q_rows.shape
    H_kv = np.asarray(k_pool).shape[2]
    r = H_q // H_kv
    out = np.zeros((N, H_q, np.asarray(v_pool).shape[3]), dtype=np.float64)
    for b, length in enumerate(np.asarray(seq_lens)):
        n = int(cu[b + 1] - cu[b])
        if n == 0:
            continue
        L = int(length)
        K = to_f64(gather_logical(k_pool, block_table, b, L, block_size), dtype)
        V = to_f64(gather_logical(v_pool, block_table, b, L, block_size), dtype)
        Q = to_f64(q_rows[cu[b]:cu[b] + n], dtype)
        for h in range(H_q):
            out[cu[b]:cu[b] + n, h] = causal_attention(Q[:, h], K[:, h // r], V[:, h // r],
                                                      past_len=L - n, scale=scale)
    return out
