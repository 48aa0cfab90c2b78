"""GPU parity of the INT8 cache path against the fp64 oracle.

The append is compared bit for bit (codes and V scales over the whole
buffers) with ``oracle.append_paged_int8``; the decode output elementwise
within the contract tolerance with ``oracle.decode_attn_paged_int8`` over
the same stored codes and scales.
"""

import zlib

import numpy as np
import pytest
import torch

import oracle
from contract import assert_contract
from gpu_util import down_bits, down_f64, log, up
from workloads import make_config_inputs, make_paged_decode_int8

pytestmark = pytest.mark.gpu

kvd = pytest.importorskip("kv_cache_decode_02_amd")


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


class Int8Dev:
    def __init__(self, inp):
        self.inp = inp
        self.q = up(inp.q)
        self.kq = up(inp.kq_pool)
        self.vq = up(inp.vq_pool)
        self.vs = up(inp.vs_pool)
        self.ks = up(inp.k_scale)
        self.k_new = up(inp.k_new)
        self.v_new = up(inp.v_new)
        self.table = up(inp.block_table)
        self.seq = up(inp.seq_lens)

    def append(self):
        kvd.kv_append_paged_int8(self.kq, self.vq, self.vs, self.k_new, self.v_new, self.ks,
                                 self.table, self.seq)


def _oracle_step(inp):
    kq, vq, vs = oracle.append_paged_int8(inp.kq_pool, inp.vq_pool, inp.vs_pool, inp.k_new,
                                          inp.v_new, "bf16", inp.k_scale, inp.block_table,
                                          inp.seq_lens)
    return kq, vq, vs


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint8)


APPEND_CASES = [
    ("gqa-d128", dict(B=5, H_q=32, H_kv=8, d=128, lens=[1, 16, 17, 500, 4096])),
    ("mha-d64", dict(B=3, H_q=4, H_kv=4, d=64, lens=[32, 33, 2])),
    ("d32", dict(B=2, H_q=2, H_kv=2, d=32, lens=[129, 7])),
]


@pytest.mark.parametrize("name,c", APPEND_CASES, ids=[n for n, _ in APPEND_CASES])
def test_append_int8_bit_exact(name, c):
    log(f"int8 append {name}")
    inp = make_paged_decode_int8(np.random.default_rng(zlib.crc32(name.encode())), c["B"],
                                 c["H_q"], c["H_kv"], c["d"], c["lens"])
    dev = Int8Dev(inp)
    dev.append()
    torch.cuda.synchronize()
    kq, vq, vs = _oracle_step(inp)
    assert np.array_equal(_bits(down_bits(dev.kq)), _bits(kq))
    assert np.array_equal(_bits(down_bits(dev.vq)), _bits(vq))
    assert np.array_equal(_bits(down_bits(dev.vs)), _bits(vs))


def test_append_int8_from_f32_rows_with_ties_and_clips():
    # fp32 rows built to hit exact half steps of the K scales (ties round to
    # even) and values beyond the calibrated range (clip to +-127).
    log("int8 append f32 ties")
    rng = np.random.default_rng(3)
    B, H_kv, d = 2, 2, 32
    inp = make_paged_decode_int8(rng, B, 4, H_kv, d, [20, 3])
    ks = np.full((H_kv, d), 0.125, np.float32)
    steps = rng.integers(-140, 141, size=(B, H_kv, d)).astype(np.float32) + 0.5
    k_new = (steps * ks).astype(np.float32)
    v_new = rng.standard_normal((B, H_kv, d)).astype(np.float32)
    v_new[0, 0] = 0.0  # a zero row: scale 0, codes 0
    dev = Int8Dev(inp)
    kvd.kv_append_paged_int8(dev.kq, dev.vq, dev.vs, up(k_new), up(v_new), up(ks), dev.table,
                             dev.seq)
    torch.cuda.synchronize()
    kq, vq, vs = oracle.append_paged_int8(inp.kq_pool, inp.vq_pool, inp.vs_pool, k_new, v_new,
                                          "f32", ks, inp.block_table, inp.seq_lens)
    assert np.array_equal(_bits(down_bits(dev.kq)), _bits(kq))
    assert np.array_equal(_bits(down_bits(dev.vq)), _bits(vq))
    assert np.array_equal(_bits(down_bits(dev.vs)), _bits(vs))


DECODE_CASES = [
    ("gqa-r4-ragged", dict(B=6, H_q=32, H_kv=8, d=128, lens=[1, 15, 17, 511, 3000, 4096], pt=0)),
    ("gqa-r4-pt256", dict(B=4, H_q=32, H_kv=8, d=128, lens=[16, 513, 2049, 100], pt=256)),
    ("mha-d128", dict(B=2, H_q=8, H_kv=8, d=128, lens=[1000, 77], pt=0)),
    ("r2-d64", dict(B=3, H_q=8, H_kv=4, d=64, lens=[33, 999, 1], pt=0)),
    ("r8-d128", dict(B=2, H_q=64, H_kv=8, d=128, lens=[2500, 300], pt=0)),
    ("mqa-d32", dict(B=2, H_q=4, H_kv=1, d=32, lens=[129, 640], pt=64)),
    # head_dim 64 on the MFMA flavour: a group of 4, and one of 16 over long
    # fixed partitions
    ("r4-d64", dict(B=3, H_q=8, H_kv=2, d=64, lens=[70, 1500, 3000], pt=0)),
    ("r16-d64-pt512", dict(B=2, H_q=16, H_kv=1, d=64, lens=[1200, 5000], pt=512)),
]


@pytest.mark.parametrize("name,c", DECODE_CASES, ids=[n for n, _ in DECODE_CASES])
def test_decode_int8_parity(name, c):
    log(f"int8 decode {name}")
    inp = make_paged_decode_int8(np.random.default_rng(zlib.crc32(name.encode()) + 9), c["B"],
                                 c["H_q"], c["H_kv"], c["d"], c["lens"])
    dev = Int8Dev(inp)
    dev.append()
    out = kvd.decode_attn_paged_int8(dev.q, dev.kq, dev.vq, dev.ks, dev.vs, dev.table, dev.seq,
                                     inp.max_seq_len, partition_tokens=c["pt"])
    torch.cuda.synchronize()
    kq, vq, vs = _oracle_step(inp)
    ref = oracle.decode_attn_paged_int8(inp.q, kq, vq, vs, inp.k_scale, inp.block_table,
                                        inp.seq_lens, "bf16")
    rep = assert_contract(down_f64(out), ref, name)
    log(f"  max_err {rep['max_err']:.3e} scaled {rep['scaled']:.3e}")


def test_int8_phases_equal_single_call():
    log("int8 partials + merge")
    inp = make_paged_decode_int8(np.random.default_rng(21), 4, 32, 8, 128, [900, 40, 2049, 16])
    dev = Int8Dev(inp)
    dev.append()
    one = kvd.decode_attn_paged_int8(dev.q, dev.kq, dev.vq, dev.ks, dev.vs, dev.table, dev.seq,
                                     inp.max_seq_len)
    ws = kvd.alloc_workspace(inp.B, 32, 8, 128, inp.max_seq_len)
    kvd.decode_attn_paged_int8_partials(dev.q, dev.kq, dev.vq, dev.ks, dev.vs, dev.table,
                                        dev.seq, inp.max_seq_len, ws)
    two = torch.empty_like(dev.q)
    kvd.decode_attn_merge(two, dev.seq, 8, inp.max_seq_len, ws)
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int16), two.view(torch.int16))


LARGE_V_CASES = [("gqa-r4", dict(H_q=32, H_kv=8)), ("mha", dict(H_q=8, H_kv=8))]


@pytest.mark.parametrize("name,c", LARGE_V_CASES, ids=[n for n, _ in LARGE_V_CASES])
def test_decode_int8_large_v_rows(name, c):
    # History V scales times 2^13: V magnitudes up to ~2.4e4, and weight times
    # V scale products up to 2^8 * 192 = 49152, inside the fp16 operand range
    # (65504) that the one-byte decode documents for them.
    log(f"int8 decode large V rows {name}")
    inp = make_paged_decode_int8(np.random.default_rng(zlib.crc32(name.encode()) + 31), 3,
                                 c["H_q"], c["H_kv"], 128, [40, 1500, 4096])
    inp.vs_pool = (inp.vs_pool * np.float32(2.0 ** 13)).astype(np.float32)
    owned = np.isin(np.arange(inp.num_blocks), inp.block_table)
    assert np.nanmax(inp.vs_pool[owned]) > 150.0
    dev = Int8Dev(inp)
    dev.append()
    out = kvd.decode_attn_paged_int8(dev.q, dev.kq, dev.vq, dev.ks, dev.vs, dev.table, dev.seq,
                   inp.max_seq_len)
    torch.cuda.synchronize()
    kq, vq, vs = _oracle_step(inp)
    ref = oracle.decode_attn_paged_int8(inp.q, kq, vq, vs, inp.k_scale, inp.block_table,
                      inp.seq_lens, "bf16")
    assert np.max(np.abs(ref)) > 100.0
    got = down_f64(out)
    assert np.all(np.isfinite(got))
    # The output is linear in V: compared in units of the factor, which is
    # the contract for the same inputs with the unscaled V (2^13 is exact).
    rep = assert_contract(got / 2.0 ** 13, ref / 2.0 ** 13, name)
    log(f"  max_err {rep['max_err']:.3e} scaled {rep['scaled']:.3e}")


def test_int8_full_size_sampled():
    name = "gqa_llama3_8b_int8"
    log(f"full {name}: generating")
    inp = make_config_inputs(name)[0]
    dev = Int8Dev(inp)
    log(f"full {name}: running ({inp.kv_bytes_read / 1e9:.2f} GB)")
    dev.append()
    out = kvd.decode_attn_paged_int8(dev.q, dev.kq, dev.vq, dev.ks, dev.vs, dev.table, dev.seq,
                                     inp.max_seq_len)
    torch.cuda.synchronize()
    got = down_f64(out)
    assert np.all(np.isfinite(got))
    kq, vq, vs = _oracle_step(inp)
    r = inp.H_q // inp.H_kv
    rng = np.random.default_rng(2)
    picks = [(0, 0), (inp.B - 1, inp.H_kv - 1)] + [
        (int(rng.integers(inp.B)), int(rng.integers(inp.H_kv))) for _ in range(4)]
    for b, g in picks:
        n = int(inp.seq_lens[b])
        K = oracle.dequantize_k(oracle.gather_logical(kq[:, :, g:g + 1], inp.block_table, b, n),
                                inp.k_scale[g:g + 1])
        V = oracle.dequantize_v(oracle.gather_logical(vq[:, :, g:g + 1], inp.block_table, b, n),
                                oracle.gather_logical(vs[:, :, g:g + 1], inp.block_table, b, n))
        q = oracle.to_f64(inp.q[b, g * r:(g + 1) * r], "bf16")
        assert_contract(got[b, g * r:(g + 1) * r], oracle.decode_attention(q, K, V),
                        f"{name} b={b} g={g}")
    log(f"full {name}: ok")
