"""The five decode workloads, by name, with their seeds.

  tiny            2 layers, H_q = H_kv = 4, d_head = 32, batch 1, 128 cached
                  tokens + 1 appended (length 129), fp32 N(0,1), contiguous
                  cache (identity block table)
  mha_llama2_7b   H_q = H_kv = 32, d_head = 128, batch 16, every length 4096,
                  bf16 N(0,1), randomly placed 16-token blocks
  gqa_llama3_8b   H_q = 32, H_kv = 8, d_head = 128, batch 64, lengths uniform
                  integers in [512, 8192], bf16 N(0,1), randomly placed blocks
  long_gqa_split  H_q = 64, H_kv = 8, d_head = 128, batch 4, lengths
                  32768 / 65536 / 98304 / 131072, bf16 N(0,1), split into
                  512-token partitions merged by log-sum-exp
  mla_deepseek_v2 absorbed MLA, 128 query heads, latent 512 + RoPE key 64
                  (576 bf16 per token), batch 32, every length 4096, q and
                  latent N(0, (1/24)^2), output in latent space (512)
  gqa_llama3_8b_int8
                  the gqa_llama3_8b batch (same seed, so the same lengths)
                  over an INT8 cache: per-channel K and per-token V scales,
                  bf16 queries and output
  gqa_llama3_8b_fp8
                  the same batch over an FP8 (E4M3) cache with the same
                  scale layout
  prefill_llama3_8b
                  chunked prefill on the Llama-3-8B shape (H_q = 32, H_kv =
                  8, d_head = 128): 4 sequences with 0 / 2048 / 4096 / 6144
                  cached positions each take a 2048-token chunk, bf16 N(0,1)

Seeds: config k (1..5 in the order above, 6 for the prefill) uses numpy
default_rng(42 + k), the INT8 and FP8 batches the GQA batch's seed; 42
is the seed of the pages' own numpy sketch.  Lengths are drawn first, then the
generator's fixed draw order (``workloads.gen``).
"""

import numpy as np

from .gen import (make_mla, make_paged_decode, make_paged_decode_fp8, make_paged_decode_int8,
                  make_paged_prefill)

CONFIGS = {
    "tiny": dict(index=1, kind="paged", B=1, H_q=4, H_kv=4, d=32, layers=2,
                 lens=("fixed", 129), dtype="f32", table="identity", std=1.0,
                 partition=0),
    "mha_llama2_7b": dict(index=2, kind="paged", B=16, H_q=32, H_kv=32, d=128, layers=1,
                          lens=("fixed", 4096), dtype="bf16", table="permuted", std=1.0,
                          partition=0),
    "gqa_llama3_8b": dict(index=3, kind="paged", B=64, H_q=32, H_kv=8, d=128, layers=1,
                          lens=("uniform", 512, 8192), dtype="bf16", table="permuted",
                          std=1.0, partition=0),
    "long_gqa_split": dict(index=4, kind="paged", B=4, H_q=64, H_kv=8, d=128, layers=1,
                           lens=("list", (32768, 65536, 98304, 131072)), dtype="bf16",
                           table="permuted", std=1.0, partition=512),
    "mla_deepseek_v2": dict(index=5, kind="mla", B=32, H=128, d_c=512, d_rope=64, layers=1,
                            lens=("fixed", 4096), dtype="bf16", table="permuted",
                            std=1.0 / 24.0, partition=0),
    "gqa_llama3_8b_int8": dict(index=3, kind="paged_int8", B=64, H_q=32, H_kv=8, d=128,
                               layers=1, lens=("uniform", 512, 8192), dtype="int8",
                               table="permuted", std=1.0, partition=0),
    "gqa_llama3_8b_fp8": dict(index=3, kind="paged_fp8", B=64, H_q=32, H_kv=8, d=128,
                              layers=1, lens=("uniform", 512, 8192), dtype="fp8",
                              table="permuted", std=1.0, partition=0),
    "prefill_llama3_8b": dict(index=6, kind="prefill", B=4, H_q=32, H_kv=8, d=128, layers=1,
                              lens=("list", (0, 2048, 4096, 6144)), new=2048, dtype="bf16",
                              table="permuted", std=1.0, partition=0),
}


def config(name):
    if name not in CONFIGS:
        raise KeyError(f"unknown workload {name!r}; choose from {sorted(CONFIGS)}")
    return dict(CONFIGS[name])


def seed_of(name):
    return 42 + config(name)["index"]


def draw_lengths(rng, spec, B):
    kind = spec[0]
    if kind == "fixed":
        return np.full(B, spec[1], dtype=np.int64)
    if kind == "list":
        if len(spec[1]) != B:
            raise ValueError("length list does not match the batch")
        return np.asarray(spec[1], dtype=np.int64)
    if kind == "uniform":
        return rng.integers(spec[1], spec[2], size=B, endpoint=True)
    raise ValueError(f"unknown length spec {spec!r}")


def make_config_inputs(name, sentinel="nan", rng=None):
    """Inputs of a named workload: a list with one entry per layer."""
    cfg = config(name)
    rng = rng if rng is not None else np.random.default_rng(seed_of(name))
    layers = []
    for _ in range(cfg["layers"]):
        B = cfg["B"]
        lens = draw_lengths(rng, cfg["lens"], B)
        if cfg["kind"] == "paged":
            layers.append(make_paged_decode(rng, B, cfg["H_q"], cfg["H_kv"], cfg["d"], lens,
                                            dtype=cfg["dtype"], table=cfg["table"],
                                            std=cfg["std"], sentinel=sentinel))
        elif cfg["kind"] == "prefill":
            layers.append(make_paged_prefill(rng, B, cfg["H_q"], cfg["H_kv"], cfg["d"], lens,
                                             [cfg["new"]] * B, dtype=cfg["dtype"],
                                             table=cfg["table"], std=cfg["std"],
                                             sentinel=sentinel))
        elif cfg["kind"] in ("paged_int8", "paged_fp8"):
            gen = make_paged_decode_int8 if cfg["kind"] == "paged_int8" else make_paged_decode_fp8
            layers.append(gen(rng, B, cfg["H_q"], cfg["H_kv"], cfg["d"], lens, table=cfg["table"],
                              std=cfg["std"], sentinel=sentinel))
        else:
            layers.append(make_mla(rng, B, cfg["H"], cfg["d_c"], cfg["d_rope"], lens,
                                   std=cfg["std"], table=cfg["table"], sentinel=sentinel))
    return layers
