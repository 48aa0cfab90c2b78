"""KVD_VALIDATE=1 on the GPU: calls whose preconditions hold give the same
bits as without the checks; a visible table entry outside the pool, an
append into a shared block, or a non-finite query is refused before any
kernel runs (the workspace and cache stay untouched)."""

import os

import numpy as np
import pytest
import torch

from gpu_util import Paged, log
from workloads import make_paged_decode

pytestmark = pytest.mark.gpu

kvd = pytest.importorskip("kv_cache_decode_02_amd")


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture
def validating():
    old = os.environ.get("KVD_VALIDATE")
    os.environ["KVD_VALIDATE"] = "1"
    yield
    if old is None:
        os.environ.pop("KVD_VALIDATE", None)
    else:
        os.environ["KVD_VALIDATE"] = old


def _inputs():
    inp = make_paged_decode(np.random.default_rng(21), 3, 8, 2, 128, [40, 17, 300])
    return inp, Paged(inp)


def test_valid_calls_are_unchanged(validating):
    log("validate: valid calls")
    inp, dev = _inputs()
    kvd.kv_append_paged(dev.k_cache, dev.v_cache, dev.k_new, dev.v_new, dev.table, dev.seq)
    checked = kvd.decode_attn_paged(dev.q, dev.k_cache, dev.v_cache, dev.table, dev.seq,
                                    inp.max_seq_len)
    torch.cuda.synchronize()
    del os.environ["KVD_VALIDATE"]
    plain = kvd.decode_attn_paged(dev.q, dev.k_cache, dev.v_cache, dev.table, dev.seq,
                                  inp.max_seq_len)
    torch.cuda.synchronize()
    assert torch.equal(checked.view(torch.int16), plain.view(torch.int16))


def test_out_of_pool_entry_is_refused(validating):
    log("validate: table entry outside the pool")
    inp, dev = _inputs()
    table = dev.table.clone()
    table[2, 3] = inp.num_blocks + 5
    ws = kvd.alloc_workspace(3, 8, 2, 128, inp.max_seq_len)
    ws.fill_(7.0)
    with pytest.raises(kvd.KvdError):
        kvd.decode_attn_paged_partials(dev.q, dev.k_cache, dev.v_cache, table, dev.seq,
                                       inp.max_seq_len, ws)
    torch.cuda.synchronize()
    assert bool((ws == 7.0).all())


def test_append_into_a_shared_block_is_refused(validating):
    log("validate: append into a shared block")
    inp, dev = _inputs()
    table = dev.table.clone()
    table[0, 2] = table[1, 1]        # sequence 0's last block is sequence 1's last block
    k_before = dev.k_cache.clone()
    with pytest.raises(kvd.KvdError):
        kvd.kv_append_paged(dev.k_cache, dev.v_cache, dev.k_new, dev.v_new, table, dev.seq)
    torch.cuda.synchronize()
    assert torch.equal(dev.k_cache.view(torch.int16), k_before.view(torch.int16))


def test_non_finite_query_is_refused(validating):
    log("validate: non-finite query")
    inp, dev = _inputs()
    q = dev.q.clone()
    q[1, 3, 5] = float("nan")
    with pytest.raises(kvd.KvdError):
        kvd.decode_attn_paged(q, dev.k_cache, dev.v_cache, dev.table, dev.seq, inp.max_seq_len)


def test_mla_fused_append_checks(validating):
    # The fused MLA append: a valid call gives the same bits as without the
    # checks; a non-finite new latent row, or a new row that lands in a block
    # another sequence also reads, is refused and the cache stays untouched.
    log("validate: fused MLA append")
    from workloads import make_mla
    from gpu_util import up
    inp = make_mla(np.random.default_rng(22), 2, 16, 512, 64, [40, 100], std=1.0)
    q, table, seq = up(inp.q), up(inp.block_table), up(inp.seq_lens)
    c_new = up(inp.c_new)
    c1, c2 = up(inp.c_pool), up(inp.c_pool)
    checked = kvd.decode_attn_mla_append(q, c1, c_new, table, seq, inp.max_seq_len)
    torch.cuda.synchronize()
    del os.environ["KVD_VALIDATE"]
    plain = kvd.decode_attn_mla_append(q, c2, c_new, table, seq, inp.max_seq_len)
    torch.cuda.synchronize()
    assert torch.equal(checked.view(torch.int16), plain.view(torch.int16))
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))
    os.environ["KVD_VALIDATE"] = "1"
    fresh = up(inp.c_pool)
    before = fresh.clone()
    bad_row = c_new.clone()
    bad_row[1, 7] = float("inf")
    with pytest.raises(kvd.KvdError):
        kvd.decode_attn_mla_append(q, fresh, bad_row, table, seq, inp.max_seq_len)
    shared = table.clone()
    shared[0, 2] = shared[1, 3]      # sequence 0's last block is one sequence 1 reads
    with pytest.raises(kvd.KvdError):
        kvd.decode_attn_mla_append(q, fresh, c_new, shared, seq, inp.max_seq_len)
    torch.cuda.synchronize()
    assert torch.equal(fresh.view(torch.int16), before.view(torch.int16))
