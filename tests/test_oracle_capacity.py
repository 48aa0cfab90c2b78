"""Pins of the oracle's byte accounting against the pages' printed numbers."""

import json
import os

import pytest

import oracle


@pytest.fixture(scope="module")
def cap(golden_dir):
    return json.load(open(os.path.join(golden_dir, "capacity.json")))


def test_per_token(cap):
    for row in cap["per_token"]:
        got = oracle.bytes_per_token(row["layers"], row["kv_heads"], row["head_dim"],
                                     row["element_bytes"])
        assert got == row["bytes"], row["source"]


def test_paged_ledgers(cap):
    for row in cap["paged"]:
        got = oracle.paged_capacity(row["lengths"], row["layers"], row["kv_heads"],
                                    row["head_dim"], row["element_bytes"], row["block_size"])
        for key in ("useful", "paged", "slots", "tail_waste"):
            assert got[key] == row[key], (key, row["source"])
        if "padded" in row:
            assert got["padded"] == row["padded"]
        if "tail_waste_bytes" in row:
            assert got["tail_waste"] * got["per_token"] == row["tail_waste_bytes"]


def test_tail_waste_bound():
    # every non-empty request wastes fewer than b slots: waste < B (b - 1) + 1
    lens = [1, 15, 16, 17, 31, 32, 33, 1000, 4097]
    got = oracle.paged_capacity(lens, 1, 1, 1, 1, 16)
    assert got["tail_waste"] <= len(lens) * 15
    assert got["slots"] == sum(-(-n // 16) * 16 for n in lens)


def test_shared_blocks(cap):
    row = cap["shared"]
    assert oracle.unique_block_bytes(row["block_tables"], row["per_token"],
                                     row["block_size"]) == row["unique_bytes"]
    entries = sum(len(t) for t in row["block_tables"])
    assert entries * row["block_size"] * row["per_token"] == row["naive_bytes"]


def test_whole_cache(cap):
    for row in cap["whole_cache"]:
        got = oracle.kv_cache_bytes(row["seq_len"], row["layers"], row["kv_heads"],
                                    row["head_dim"], row["element_bytes"], row["batch"])
        assert got == row["bytes"], row["source"]


def test_misprinted_scenario_is_not_a_pin(cap):
    row = cap["misprint"]
    got = oracle.kv_cache_bytes(row["seq_len"], row["layers"], row["kv_heads"],
                                row["head_dim"], row["element_bytes"], row["batch"])
    assert got == row["formula"] == 2 * row["printed"]


def test_mla_elements(cap):
    m = cap["mla"]
    n = oracle.mla_elements_per_token(m["d_c"], m["d_rope"])
    assert n == m["elements"]
    assert 2 * m["mha_heads"] * m["d_h"] == m["mha_elements"]
    assert round(m["mha_elements"] / n) == m["ratio_inverse_rounded"]
    assert n / (2 * m["d_h"]) == m["gqa_groups"]


def test_validation():
    with pytest.raises(ValueError):
        oracle.paged_capacity([3, -1], 1, 1, 1, 1, 16)
    with pytest.raises(ValueError):
        oracle.paged_capacity([3.0], 1, 1, 1, 1, 16)
    with pytest.raises(ValueError):
        oracle.paged_capacity([3], 0, 1, 1, 1, 16)
    with pytest.raises(ValueError):
        oracle.paged_capacity([3], 1, 1, 1, 1, 0)
    assert oracle.paged_capacity([], 1, 1, 1, 1, 16)["padded"] == 0
