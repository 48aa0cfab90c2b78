"""Paged decode attention for MI355X (gfx950): Python face of libkvdecode.so.

One decode step of one layer: ``kv_append_paged`` writes the step's K/V row
into the paged cache, ``decode_attn_paged`` attends over the whole visible
history (split-KV partials, then a log-sum-exp merge), and
``decode_attn_paged_append`` does both in one pass; ``kv_append_paged_int8``
and ``decode_attn_paged_int8`` are the same step over an INT8 cache (K scaled
per channel, V per token), the ``_fp8`` functions over an FP8 (E4M3) cache; ``decode_attn_mla`` is the absorbed multi-head
latent attention variant over a latent cache.  The functions mirror
the C ABI in ``include/kvdecode.h`` and only marshal arguments; importing this
package fails if the HIP library has not been built.
"""

from ._native import (
    KvdError,
    kv_append_paged,
    decode_attn_paged,
    decode_attn_paged_partials,
    decode_attn_paged_append,
    decode_attn_paged_append_partials,
    decode_attn_paged_append_noalloc,
    decode_attn_noalloc_scratch_bytes,
    stream_read,
    stream_read_sink_bytes,
    lds_read,
    lds_read_sink_bytes,
    lds_read_bytes,
    decode_attn_paged_window,
    decode_attn_paged_window_partials,
    decode_attn_merge,
    decode_attn_workspace_bytes,
    decode_attn_partition_tokens,
    alloc_workspace,
    decode_attn_mla,
    decode_attn_mla_partials,
    decode_attn_mla_append,
    decode_attn_mla_append_partials,
    mla_default_scale,
    kv_append_paged_int8,
    decode_attn_paged_int8,
    decode_attn_paged_int8_partials,
    kv_append_paged_fp8,
    decode_attn_paged_fp8,
    decode_attn_paged_fp8_partials,
    kv_copy_blocks,
    kv_append_paged_multi,
    prefill_attn_paged,
    block_hashes,
    BlockPool,
    PoolExhausted,
    validate_tables,
    validate_finite,
    LIB_PATH,
    HEADER_PATH,
)

__all__ = [
    "KvdError", "kv_append_paged", "decode_attn_paged", "decode_attn_paged_partials",
    "decode_attn_paged_append", "decode_attn_paged_append_partials",
    "decode_attn_paged_append_noalloc", "decode_attn_noalloc_scratch_bytes",
    "stream_read", "stream_read_sink_bytes", "lds_read", "lds_read_sink_bytes", "lds_read_bytes",
    "decode_attn_paged_window", "decode_attn_paged_window_partials",
    "decode_attn_merge", "decode_attn_workspace_bytes", "decode_attn_partition_tokens",
    "alloc_workspace", "decode_attn_mla", "decode_attn_mla_partials",
    "decode_attn_mla_append", "decode_attn_mla_append_partials", "mla_default_scale",
    "kv_append_paged_int8", "decode_attn_paged_int8", "decode_attn_paged_int8_partials",
    "kv_append_paged_fp8", "decode_attn_paged_fp8", "decode_attn_paged_fp8_partials",
    "kv_copy_blocks", "kv_append_paged_multi", "prefill_attn_paged", "block_hashes",
    "BlockPool", "PoolExhausted", "validate_tables", "validate_finite",
    "LIB_PATH", "HEADER_PATH",
]
