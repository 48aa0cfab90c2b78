"""The seeded input generator: determinism, layout and sentinels (CPU only)."""

import numpy as np
import pytest
import torch

from workloads import (make_paged_decode, make_mla, bf16_round_bits, make_config_inputs,
                       config, UNUSED_TABLE_ENTRY)
from workloads.configs import draw_lengths, seed_of


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100_000).astype(np.float32),
        (rng.standard_normal(1000) * 1e-30).astype(np.float32),
        np.array([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 0.0, -0.0, 65504.0, 3.0e38],
                 dtype=np.float32),
    ])
    ours = bf16_round_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_deterministic():
    a = make_paged_decode(np.random.default_rng(5), 3, 8, 2, 16, [5, 40, 17])
    b = make_paged_decode(np.random.default_rng(5), 3, 8, 2, 16, [5, 40, 17])
    for f in ("q", "k_pool", "v_pool", "k_new", "v_new", "block_table"):
        assert np.array_equal(getattr(a, f).view(np.uint8), getattr(b, f).view(np.uint8))


@pytest.mark.parametrize("table", ["permuted", "identity"])
def test_layout_and_sentinels(table):
    lens = [1, 15, 16, 17, 32, 33, 100]
    inp = make_paged_decode(np.random.default_rng(1), len(lens), 4, 2, 8, lens, table=table)
    need = [-(-n // 16) for n in lens]
    assert inp.num_blocks == sum(need)
    assert inp.k_pool.shape == (inp.num_blocks, 16, 2, 8)
    used = np.concatenate([inp.block_table[b, :need[b]] for b in range(len(lens))])
    assert sorted(used.tolist()) == list(range(inp.num_blocks))
    for b, n in enumerate(need):
        assert np.all(inp.block_table[b, n:] == UNUSED_TABLE_ENTRY)
    if table == "identity":
        assert used.tolist() == list(range(inp.num_blocks))
    # history slots are finite; this step's slot and the tail hold NaN
    for b, n in enumerate(lens):
        for t in range(need[b] * 16):
            blk = inp.block_table[b, t // 16]
            row = inp.k_pool[blk, t % 16].view(np.uint16)
            is_nan = np.all(row == 0x7FC0)
            assert is_nan == (t >= n - 1), (b, t)


def test_zero_sentinel_for_timing():
    inp = make_paged_decode(np.random.default_rng(2), 2, 4, 4, 8, [3, 20], sentinel="zero",
                            dtype="f32")
    assert np.all(np.isfinite(inp.k_pool)) and np.all(np.isfinite(inp.v_pool))


def test_config_shapes_small():
    tiny = make_config_inputs("tiny")
    assert len(tiny) == 2
    for layer in tiny:
        assert layer.dtype == "f32" and layer.seq_lens.tolist() == [129]
        assert layer.block_table.tolist() == [list(range(9))]
        assert layer.q.shape == (1, 4, 32) and layer.k_pool.shape == (9, 16, 4, 32)
    assert not np.array_equal(tiny[0].q, tiny[1].q)


def test_gqa_lengths_drawn_from_seed():
    cfg = config("gqa_llama3_8b")
    lens = draw_lengths(np.random.default_rng(seed_of("gqa_llama3_8b")), cfg["lens"], cfg["B"])
    assert lens.min() >= 512 and lens.max() <= 8192
    assert np.any(lens % 16 != 0)


def test_mla_layout():
    inp = make_mla(np.random.default_rng(3), 2, 16, 512, 64, [5, 33], std=1 / 24)
    assert inp.q.shape == (2, 16, 576) and inp.c_pool.shape == (inp.num_blocks, 16, 576)
    assert inp.num_blocks == 1 + 3
    assert inp.kv_bytes_read == (5 + 33) * 576 * 2
