"""Plain fp64 CPU oracle for paged decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, constants or
helpers with the HIP library in ``kv_cache_decode_02_amd``; the only module
both sides use is ``workloads`` (seeded synthetic inputs, no attention maths).

Everything here is written from the definitions on four web pages about the
KV cache.  Citation keys used in this package:

  [DQ]  "KV-Cache——为什么AI回复越来越快，不用从头算一遍？" (dataqian.wang)
  [LC]  "KV Cache（键值缓存）" (LLM Compass, inference/kv-cache)
  [MV]  "单请求 KV Cache" (mini-vllm tutorial, step 07)
  [SW]  "KV缓存原理与显存估算" (LLM Systems Wiki, read/kv-cache)

Modules:
  numerics   exact unpacking of stored bf16 / fp32 values to fp64
  paged      slot mapping, in-place append and logical gather (block table)
  attention  single-query decode attention, sliding-window decode, split
             partials + LSE merge, absorbed MLA, full causal recompute
  capacity   KV byte accounting (per token, useful / padded / paged, shared)
  quant      INT8 cache: per-channel K / per-token V codes, append, decode
  quant_fp8  FP8 (E4M3) cache: the same scales over E4M3 codes
  allocator  block pool model: counts, fork, copy-on-write, chained keys

Pins: every function is checked in ``tests/test_oracle_*.py`` against values
printed on the pages (``tests/golden/``), closed forms, invariants and special
cases.  No function here is "parity unpinned".
"""

from .numerics import bf16_bits_to_f64, to_f64
from .paged import slot_of, append_paged, append_paged_multi, gather_history, gather_logical
from .attention import (
    decode_attention,
    decode_attention_weights,
    decode_attn_paged,
    window_start,
    decode_attn_paged_window,
    split_partials,
    lse_merge,
    decode_attention_split,
    mla_decode,
    mla_decode_paged,
    causal_attention,
    prefill_attn_paged,
)
from .quant import (
    quantize,
    channel_scales,
    append_paged_int8,
    dequantize_k,
    dequantize_v,
    decode_attn_paged_int8,
)
from .quant_fp8 import (
    e4m3_value,
    e4m3_decode,
    e4m3_encode,
    quantize_fp8,
    channel_scales_fp8,
    append_paged_fp8,
    decode_attn_paged_fp8,
)
from .allocator import block_hashes, BlockPool, PoolExhausted
from .capacity import (
    bytes_per_token,
    paged_capacity,
    unique_block_bytes,
    kv_cache_bytes,
    mla_elements_per_token,
)

__all__ = [
    "bf16_bits_to_f64", "to_f64",
    "slot_of", "append_paged", "append_paged_multi", "gather_history", "gather_logical",
    "decode_attention", "decode_attention_weights", "decode_attn_paged",
    "window_start", "decode_attn_paged_window",
    "split_partials", "lse_merge", "decode_attention_split",
    "mla_decode", "mla_decode_paged", "causal_attention", "prefill_attn_paged",
    "bytes_per_token", "paged_capacity", "unique_block_bytes",
    "kv_cache_bytes", "mla_elements_per_token",
    "quantize", "channel_scales", "append_paged_int8", "dequantize_k",
    "dequantize_v", "decode_attn_paged_int8",
    "e4m3_value", "e4m3_decode", "e4m3_encode", "quantize_fp8", "channel_scales_fp8",
    "append_paged_fp8", "decode_attn_paged_fp8",
    "block_hashes", "BlockPool", "PoolExhausted",
]
