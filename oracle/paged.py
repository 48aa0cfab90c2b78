"""Block-table slot mapping, in-place append and logical gather (oracle).

Test infrastructure only.  Citation keys are listed in ``oracle/__init__.py``.

Model of the paged cache:
  * A sequence's cache is cut into fixed blocks of ``block_size`` tokens
    (16 by default); a per-sequence block table maps logical block j to a
    physical block anywhere in the pool ([DQ] 08 "PagedAttention（vLLM）":
    logical pages map to non-contiguous physical pages through a page table;
    [LC] 2.3 "路线二：系统管理——PagedAttention 分页", default block of 16).
  * Inside a physical block the layout is token-major, ``pool[blk, off, h, j]``
    -- the per-token ``[seq, heads, d_head]`` layout of the tutorial's
    ``past_key_values`` ([MV] "past_key_values 的数据结构").  With an identity
    block table the pool is byte-for-byte the preallocated contiguous cache
    ``K_cache[max_len, heads, d_head]`` of [MV] "生产系统的做法：预分配 +
    in-place 写入".
  * ``seq_lens[b]`` is the length *after* this step's token has been appended
    ([SW] 前置知识: the cache length counts positions already forwarded;
    [SW] 知识点二: after the append K' has T+1 rows), so the new token goes to
    logical position ``seq_lens[b] - 1``.
"""

import numpy as np


def slot_of(block_table, b, pos, block_size=16):
    """Physical (block, offset) of logical position ``pos`` of sequence ``b``.

    Logical position t lives in logical block t // block_size at offset
    t % block_size; the table row of sequence b names the physical block.
    """
    if pos < 0:
        raise ValueError("position must be non-negative")
    j, off = divmod(int(pos), int(block_size))
    bt = np.asarray(block_table)
    if j >= bt.shape[1]:
        raise ValueError("position beyond the block table row")
    return int(bt[b, j]), off


def _check_block(blk, num_blocks):
    if not (0 <= blk < num_blocks):
        raise ValueError(f"block table entry {blk} outside the pool [0, {num_blocks})")


def append_paged(k_pool, v_pool, k_new, v_new, block_table, seq_lens, block_size=16):
    """Write each sequence's new K (and V) row into its slot; return new pools.

    In-place slot write of [MV] "生产系统的做法：预分配 + in-place 写入"
    (``K_cache[current_pos] = K_new``), addressed through the block table.
    The inputs are not modified: copies are returned, so a test can compare
    the whole buffer before and after.  ``v_pool`` / ``v_new`` may be None
    (a latent cache with no separate V).
    """
    k_out = np.array(k_pool, copy=True)
    v_out = None if v_pool is None else np.array(v_pool, copy=True)
    if (v_pool is None) != (v_new is None):
        raise ValueError("v_new must be given exactly when v_pool is")
    nb = k_out.shape[0]
    for b, length in enumerate(np.asarray(seq_lens)):
        if length < 1:
            raise ValueError("seq_lens must be >= 1 (the appended token is counted)")
        blk, off = slot_of(block_table, b, int(length) - 1, block_size)
        _check_block(blk, nb)
        k_out[blk, off] = k_new[b]
        if v_out is not None:
            v_out[blk, off] = v_new[b]
    return k_out, v_out


def gather_logical(pool, block_table, b, length, block_size=16):
    """Stored rows of logical positions [0, length) of sequence ``b``.

    Returns an array ``[length, ...]`` in logical token order, in the pool's
    own storage dtype (no conversion).
    """
    pool = np.asarray(pool)
    nb = pool.shape[0]
    rows = np.empty((int(length),) + pool.shape[2:], dtype=pool.dtype)
    for t in range(int(length)):
        blk, off = slot_of(block_table, b, t, block_size)
        _check_block(blk, nb)
        rows[t] = pool[blk, off]
    return rows


def gather_history(pool, block_table, seq_lens, b, block_size=16):
    """The cached history of sequence b: positions [0, seq_lens[b] - 1)."""
    return gather_logical(pool, block_table, b, int(seq_lens[b]) - 1, block_size)


def append_paged_multi(k_pool, v_pool, k_rows, v_rows, cu_rows, block_table, seq_lens,
                       block_size=16):
    """Write n_b new rows per sequence, n_b = cu_rows[b + 1] - cu_rows[b],
    into positions [seq_lens[b] - n_b, seq_lens[b]) (seq_lens counts them, as
    for the single-row append); return new pools.

    The many-slot form of the in-place write ([MV] 生产系统的做法; [SW] 知识点二:
    prefill writes the prompt's rows, decode appends one per step).  k_rows /
    v_rows: [N, H_kv, d] in row order of cu_rows.
    """
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    cu = np.asarray(cu_rows)
    nb = k_out.shape[0]
    for b, length in enumerate(np.asarray(seq_lens)):
        n = int(cu[b + 1] - cu[b])
        if n > int(length):
            raise ValueError("more new rows than positions")
        for i in range(n):
            blk, off = slot_of(block_table, b, int(length) - n + i, block_size)
            _check_block(blk, nb)
            k_out[blk, off] = k_rows[cu[b] + i]
            v_out[blk, off] = v_rows[cu[b] + i]
    return k_out, v_out
