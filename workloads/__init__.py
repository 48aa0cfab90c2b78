"""Seeded synthetic inputs for paged decode attention.

This module is the only code that both the oracle side (tests) and the HIP
side (tests, bench) use.  It draws random numbers and lays them out; it holds
none of the attention arithmetic.  No model weights, datasets or benchmark
suites are involved: the tensors are shaped like the pages' Llama-2-7B,
Llama-3-8B and DeepSeek-V2 examples and filled from a seeded generator.
"""

from .gen import (
    PagedDecodeInputs,
    MlaInputs,
    bf16_round_bits,
    make_paged_decode,
    PagedInt8Inputs,
    make_paged_decode_int8,
    make_paged_decode_fp8,
    PagedPrefillInputs,
    make_paged_prefill,
    make_mla,
    BLOCK_SIZE,
    UNUSED_TABLE_ENTRY,
)
from .configs import CONFIGS, config, make_config_inputs

__all__ = [
    "PagedDecodeInputs", "MlaInputs", "bf16_round_bits", "make_paged_decode",
    "PagedInt8Inputs", "make_paged_decode_int8", "make_paged_decode_fp8", "PagedPrefillInputs",
    "make_paged_prefill",
    "make_mla", "BLOCK_SIZE", "UNUSED_TABLE_ENTRY", "CONFIGS", "config",
    "make_config_inputs",
]
