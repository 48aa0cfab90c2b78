"""Pins of the oracle's block-table mapping, append and gather (CPU only)."""

import numpy as np
import pytest

import oracle
from workloads import make_paged_decode, UNUSED_TABLE_ENTRY


def test_identity_table_is_the_contiguous_cache():
    # Appending token after token into a token-major pool through an identity
    # table writes exactly what K_cache[pos] = K_new writes into a preallocated
    # [max_len, heads, d] array.
    rng = np.random.default_rng(0)
    T, H, d, bs = 45, 3, 4, 16
    nb = -(-T // bs)
    table = np.arange(nb, dtype=np.int32)[None, :]
    rows = rng.standard_normal((T, H, d))
    pool = np.zeros((nb, bs, H, d))
    contiguous = np.zeros((nb * bs, H, d))
    for pos in range(T):
        pool, _ = oracle.append_paged(pool, None, rows[pos:pos + 1], None, table,
                                      np.array([pos + 1]), bs)
        contiguous[pos] = rows[pos]
    assert np.array_equal(pool.reshape(nb * bs, H, d), contiguous)
    assert np.array_equal(oracle.gather_logical(pool, table, 0, T, bs), rows)


def test_append_round_trip_under_permuted_table():
    rng = np.random.default_rng(1)
    T, H, d, bs = 70, 2, 8, 16
    nb = -(-T // bs) + 3  # spare blocks that nothing may touch
    table = np.full((1, 8), UNUSED_TABLE_ENTRY, dtype=np.int32)
    table[0, :-(-T // bs)] = rng.permutation(nb)[:-(-T // bs)]
    rows = rng.standard_normal((T, H, d))
    pool = np.full((nb, bs, H, d), 7.0)
    for pos in range(T):
        pool, _ = oracle.append_paged(pool, None, rows[pos:pos + 1], None, table,
                                      np.array([pos + 1]), bs)
    assert np.array_equal(oracle.gather_logical(pool, table, 0, T, bs), rows)
    used = set(table[0, :-(-T // bs)].tolist())
    for blk in range(nb):
        if blk not in used:
            assert np.all(pool[blk] == 7.0)


def test_append_touches_only_the_slot():
    rng = np.random.default_rng(2)
    inp = make_paged_decode(rng, 5, 4, 2, 8, [1, 16, 17, 33, 40], dtype="bf16")
    k2, v2 = oracle.append_paged(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new,
                                 inp.block_table, inp.seq_lens)
    changed = np.argwhere(np.any(k2.view(np.uint16) != inp.k_pool.view(np.uint16), axis=(2, 3)))
    expect = set()
    for b, n in enumerate(inp.seq_lens):
        expect.add(oracle.slot_of(inp.block_table, b, n - 1))
    assert {tuple(x) for x in changed.tolist()} == expect
    for b, n in enumerate(inp.seq_lens):
        blk, off = oracle.slot_of(inp.block_table, b, n - 1)
        assert np.array_equal(k2[blk, off], inp.k_new[b])
        assert np.array_equal(v2[blk, off], inp.v_new[b])


def test_slot_formula_examples():
    table = np.array([[5, 9, 2]], dtype=np.int32)
    assert oracle.slot_of(table, 0, 0) == (5, 0)
    assert oracle.slot_of(table, 0, 15) == (5, 15)
    assert oracle.slot_of(table, 0, 16) == (9, 0)
    assert oracle.slot_of(table, 0, 47) == (2, 15)
    with pytest.raises(ValueError):
        oracle.slot_of(table, 0, 48)


def test_block_placement_does_not_change_the_output():
    # the same logical rows placed under two different permutations give
    # bit-identical oracle outputs
    rng = np.random.default_rng(3)
    a = make_paged_decode(np.random.default_rng(10), 3, 8, 2, 16, [20, 37, 5])
    b_tab = np.full_like(a.block_table, UNUSED_TABLE_ENTRY)
    perm = rng.permutation(a.num_blocks).astype(np.int32)
    k_pool = np.empty_like(a.k_pool)
    v_pool = np.empty_like(a.v_pool)
    for b in range(a.B):
        for j in range(-(-int(a.seq_lens[b]) // 16)):
            old = a.block_table[b, j]
            b_tab[b, j] = perm[old]
            k_pool[perm[old]] = a.k_pool[old]
            v_pool[perm[old]] = a.v_pool[old]
    o1 = oracle.decode_attn_paged(a.q, a.k_pool, a.v_pool, a.block_table, a.seq_lens,
                                  "bf16", a.k_new, a.v_new)
    o2 = oracle.decode_attn_paged(a.q, k_pool, v_pool, b_tab, a.seq_lens,
                                  "bf16", a.k_new, a.v_new)
    assert np.array_equal(o1, o2)


def test_paged_after_append_equals_logical_append():
    rng = np.random.default_rng(4)
    inp = make_paged_decode(rng, 4, 8, 4, 16, [1, 16, 17, 50], dtype="bf16")
    k2, v2 = oracle.append_paged(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new,
                                 inp.block_table, inp.seq_lens)
    a = oracle.decode_attn_paged(inp.q, k2, v2, inp.block_table, inp.seq_lens, "bf16")
    b = oracle.decode_attn_paged(inp.q, inp.k_pool, inp.v_pool, inp.block_table,
                                 inp.seq_lens, "bf16", inp.k_new, inp.v_new)
    assert np.array_equal(a, b)
    assert np.all(np.isfinite(a))


def test_rejects_out_of_pool_entries():
    table = np.array([[0, UNUSED_TABLE_ENTRY]], dtype=np.int32)
    pool = np.zeros((1, 16, 1, 4))
    with pytest.raises(ValueError):
        oracle.gather_logical(pool, table, 0, 17)
    with pytest.raises(ValueError):
        oracle.append_paged(pool, None, np.zeros((1, 1, 4)), None, table, np.array([0]))
