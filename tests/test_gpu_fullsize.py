"""Every output of the benchmarked steps at full size against the fp64 oracle.

Each test runs exactly the kernels bench.py times for its workload, with the
same arguments (the partials entry point with the append fused in where the
step fuses it, then the merge), on the workload's own seeded inputs, and
compares every (sequence, query head) output row with the oracle's decode
attention ("KV缓存原理与显存估算", 知识点二: z = scale q.K, a = softmax(z),
o = sum a V) over the cache after the oracle's append.  The appended slots
are compared bit for bit over the whole cache buffers.  One-byte caches go
through the oracle's quantising append and dequantisation first
("KV-Cache——为什么AI回复越来越快", KV-Cache量化).

Inputs here hold the NaN sentinel in every slot that holds no history, so a
read of a tail slot or of this step's slot before its append shows up as NaN.
"""

import numpy as np
import pytest
import torch

import oracle
from contract import assert_contract
from gpu_util import Paged, down_bits, down_f64, log, up
from workloads import config, make_config_inputs

pytestmark = pytest.mark.gpu

kvd = pytest.importorskip("kv_cache_decode_02_amd")


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _check_rows(name, got, ref_of, B, H_kv, r):
    """ref_of(b, g) -> oracle rows [r, width] of query heads g*r .. g*r+r-1."""
    worst = {"max_err": 0.0, "scaled": 0.0}
    for b in range(B):
        for g in range(H_kv):
            rep = assert_contract(got[b, g * r:(g + 1) * r], ref_of(b, g), f"{name} b={b} g={g}")
            worst["max_err"] = max(worst["max_err"], rep["max_err"])
            worst["scaled"] = max(worst["scaled"], rep["scaled"])
    log(f"  {B * H_kv} (sequence, kv head) groups, all {B * H_kv * r} rows: "
        f"max_err {worst['max_err']:.3e}, worst scaled {worst['scaled']:.3e}")


PAGED = ["mha_llama2_7b", "gqa_llama3_8b", "long_gqa_split"]


@pytest.mark.parametrize("name", PAGED)
def test_paged_step_every_output(name):
    cfg = config(name)
    pt = cfg["partition"]
    log(f"full {name}: generating")
    inp = make_config_inputs(name)[0]
    dev = Paged(inp)
    L = inp.max_seq_len
    ws = kvd.alloc_workspace(inp.B, inp.H_q, inp.H_kv, inp.d, L, pt)
    out = torch.empty_like(dev.q)
    log(f"full {name}: step (append fused into the partials kernel, merge), pt={pt}")
    kvd.decode_attn_paged_append_partials(dev.q, dev.k_cache, dev.v_cache, dev.k_new, dev.v_new,
                                          dev.table, dev.seq, L, ws, partition_tokens=pt)
    kvd.decode_attn_merge(out, dev.seq, inp.H_kv, L, ws, partition_tokens=pt)
    torch.cuda.synchronize()
    got = down_f64(out)
    log(f"full {name}: append bit for bit")
    k_ref, v_ref = oracle.append_paged(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new,
                                       inp.block_table, inp.seq_lens)
    assert np.array_equal(down_bits(dev.k_cache), k_ref)
    assert np.array_equal(down_bits(dev.v_cache), v_ref)
    del dev
    log(f"full {name}: oracle on every row")
    r = inp.H_q // inp.H_kv

    def ref_of(b, g):
        n = int(inp.seq_lens[b])
        K = oracle.to_f64(oracle.gather_logical(k_ref[:, :, g:g + 1], inp.block_table, b, n), "bf16")
        V = oracle.to_f64(oracle.gather_logical(v_ref[:, :, g:g + 1], inp.block_table, b, n), "bf16")
        return oracle.decode_attention(oracle.to_f64(inp.q[b, g * r:(g + 1) * r], "bf16"), K, V)

    _check_rows(name, got, ref_of, inp.B, inp.H_kv, r)


def test_mla_step_every_output():
    name = "mla_deepseek_v2"
    log(f"full {name}: generating")
    inp = make_config_inputs(name)[0]
    q, c = up(inp.q), up(inp.c_pool)
    c_new, table, seq = up(inp.c_new), up(inp.block_table), up(inp.seq_lens)
    L = inp.max_seq_len
    ws = kvd.alloc_workspace(inp.B, inp.H, 1, inp.d_c, L, 0)
    out = torch.empty((inp.B, inp.H, inp.d_c), dtype=torch.bfloat16, device=q.device)
    log(f"full {name}: step (append fused into the MLA partials kernel, merge)")
    kvd.decode_attn_mla_append_partials(q, c, c_new, table, seq, L, ws)
    kvd.decode_attn_merge(out, seq, 1, L, ws)
    torch.cuda.synchronize()
    got = down_f64(out)
    c_ref, _ = oracle.append_paged(inp.c_pool, None, inp.c_new, None, inp.block_table,
                                   inp.seq_lens)
    assert np.array_equal(down_bits(c), c_ref)
    scale = kvd.mla_default_scale()

    def ref_of(b, g):
        n = int(inp.seq_lens[b])
        C = oracle.to_f64(oracle.gather_logical(c_ref, inp.block_table, b, n), "bf16")
        return oracle.mla_decode(oracle.to_f64(inp.q[b], "bf16"), C, inp.d_c, scale)

    _check_rows(name, got, ref_of, inp.B, 1, inp.H)


@pytest.mark.parametrize("name", ["gqa_llama3_8b_int8", "gqa_llama3_8b_fp8"])
def test_one_byte_step_every_output(name):
    log(f"full {name}: generating")
    inp = make_config_inputs(name)[0]
    fp8 = inp.codes == "fp8"
    q, kq, vq, vs = up(inp.q), up(inp.kq_pool), up(inp.vq_pool), up(inp.vs_pool)
    ks, kn, vn = up(inp.k_scale), up(inp.k_new), up(inp.v_new)
    table, seq = up(inp.block_table), up(inp.seq_lens)
    L = inp.max_seq_len
    ws = kvd.alloc_workspace(inp.B, inp.H_q, inp.H_kv, inp.d, L, 0)
    out = torch.empty_like(q)
    append = kvd.kv_append_paged_fp8 if fp8 else kvd.kv_append_paged_int8
    partials = kvd.decode_attn_paged_fp8_partials if fp8 else kvd.decode_attn_paged_int8_partials
    log(f"full {name}: step (quantising append, partials, merge)")
    append(kq, vq, vs, kn, vn, ks, table, seq)
    partials(q, kq, vq, ks, vs, table, seq, L, ws)
    kvd.decode_attn_merge(out, seq, inp.H_kv, L, ws)
    torch.cuda.synchronize()
    got = down_f64(out)
    oracle_append = oracle.append_paged_fp8 if fp8 else oracle.append_paged_int8
    kq_ref, vq_ref, vs_ref = oracle_append(inp.kq_pool, inp.vq_pool, inp.vs_pool, inp.k_new,
                                           inp.v_new, "bf16", inp.k_scale, inp.block_table,
                                           inp.seq_lens)
    bits = lambda a: np.ascontiguousarray(a).view(np.uint8)  # noqa: E731
    assert np.array_equal(bits(down_bits(kq)), bits(kq_ref))
    assert np.array_equal(bits(down_bits(vq)), bits(vq_ref))
    assert np.array_equal(bits(down_bits(vs)), bits(vs_ref))
    # codes -> values: E4M3 decoding, or the integer codes themselves
    values = oracle.e4m3_decode if fp8 else (lambda c: np.asarray(c, dtype=np.float64))
    r = inp.H_q // inp.H_kv

    def ref_of(b, g):
        n = int(inp.seq_lens[b])
        hs = slice(g, g + 1)
        K = oracle.dequantize_k(values(oracle.gather_logical(kq_ref[:, :, hs], inp.block_table, b, n)),
                                inp.k_scale[hs])
        V = oracle.dequantize_v(values(oracle.gather_logical(vq_ref[:, :, hs], inp.block_table, b, n)),
                                oracle.gather_logical(vs_ref[:, :, hs], inp.block_table, b, n))
        return oracle.decode_attention(oracle.to_f64(inp.q[b, g * r:(g + 1) * r], "bf16"), K, V)

    _check_rows(name, got, ref_of, inp.B, inp.H_kv, r)
