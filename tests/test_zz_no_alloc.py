"""The allocation-free decode step against the workspace one (GPU).

decode_attn_paged_append_noalloc runs the kernels of decode_attn_paged_append
with the library's per-GPU scratch array in place of a caller workspace.  Two
calls in a row -- the second with a smaller batch, shorter histories and fewer
heads, so it runs over what the first left in the array -- must each give
the workspace entry point's output bit for bit, the same appended cache
slots, and the oracle's result within the contract tolerance.  The calls
must not change the device's free memory, and a call that needs more than
the scratch array is refused with nothing launched.
"""

import numpy as np
import pytest
import torch

import oracle
from contract import assert_contract
from gpu_util import Paged, down_bits, down_f64, log
from workloads import make_paged_decode

pytestmark = pytest.mark.gpu

kvd = pytest.importorskip("kv_cache_decode_02_amd")


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


CALLS = [
    # (seed, B, H_q, H_kv, d, lengths, partition_tokens)
    (71, 12, 32, 8, 128, [4096, 17, 1, 900, 2049, 16, 333, 7000, 512, 64, 3000, 1500], 0),
    (72, 3, 8, 2, 64, [40, 700, 5], 0),
    (73, 2, 16, 4, 128, [1500, 300], 256),
]


def _step_pair(seed, B, H_q, H_kv, d, lens, pt):
    inp = make_paged_decode(np.random.default_rng(seed), B, H_q, H_kv, d, lens)
    ref_dev, na_dev = Paged(inp), Paged(inp)
    L = inp.max_seq_len
    want = kvd.decode_attn_paged_append(ref_dev.q, ref_dev.k_cache, ref_dev.v_cache,
                                        ref_dev.k_new, ref_dev.v_new, ref_dev.table, ref_dev.seq,
                                        L, partition_tokens=pt)
    torch.cuda.synchronize()
    out = torch.full_like(na_dev.q, float("nan"))
    free0 = torch.cuda.mem_get_info()[0]
    kvd.decode_attn_paged_append_noalloc(na_dev.q, na_dev.k_cache, na_dev.v_cache, na_dev.k_new,
                                         na_dev.v_new, na_dev.table, na_dev.seq, L, out,
                                         partition_tokens=pt)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    return inp, want, out, ref_dev, na_dev, free0, free1


def test_two_calls_equal_the_workspace_entry_point():
    assert kvd.decode_attn_noalloc_scratch_bytes() == 64 << 20
    for i, call in enumerate(CALLS):
        log(f"noalloc call {i}: B={call[1]} H_q={call[2]} H_kv={call[3]} d={call[4]} pt={call[6]}")
        inp, want, got, ref_dev, na_dev, free0, free1 = _step_pair(*call)
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"call {i}"
        assert torch.equal(na_dev.k_cache.view(torch.int16), ref_dev.k_cache.view(torch.int16))
        assert torch.equal(na_dev.v_cache.view(torch.int16), ref_dev.v_cache.view(torch.int16))
        k_ref, v_ref = oracle.append_paged(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new,
                                           inp.block_table, inp.seq_lens)
        assert np.array_equal(down_bits(na_dev.k_cache), k_ref)
        assert np.array_equal(down_bits(na_dev.v_cache), v_ref)
        ref = oracle.decode_attn_paged(inp.q, inp.k_pool, inp.v_pool, inp.block_table,
                                       inp.seq_lens, inp.dtype, inp.k_new, inp.v_new)
        rep = assert_contract(down_f64(got), ref, f"noalloc call {i}")
        log(f"  bit-identical to the workspace call; max_err {rep['max_err']:.3e}")
        if i > 0:  # the first call may load the library's code object on this device
            assert free1 == free0, (free0, free1)


def test_oversize_call_is_refused_before_launch():
    # 8192 sequences of up to 8192 positions with 32 query heads need far
    # more partial results than the scratch array holds.
    B, H_q, H_kv, d, L = 8191, 32, 8, 128, 8192
    need = kvd.decode_attn_workspace_bytes(B, H_q, H_kv, d, L, 0)
    assert need > kvd.decode_attn_noalloc_scratch_bytes()
    dev = torch.device("cuda:0")
    q = torch.zeros((B, H_q, d), dtype=torch.bfloat16, device=dev)
    kc = torch.zeros((1, 16, H_kv, d), dtype=torch.bfloat16, device=dev)
    kn = torch.zeros((B, H_kv, d), dtype=torch.bfloat16, device=dev)
    table = torch.zeros((B, L // 16), dtype=torch.int32, device=dev)
    seq = torch.ones(B, dtype=torch.int32, device=dev)
    out = torch.full_like(q, 7.0)
    with pytest.raises(kvd.KvdError, match="workspace"):
        kvd.decode_attn_paged_append_noalloc(q, kc, kc.clone(), kn, kn.clone(), table, seq, L,
                                             out)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)  # nothing ran
