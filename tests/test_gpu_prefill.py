"""GPU parity of the many-slot append and the causal prefill kernel.

The append is compared bit for bit with ``oracle.append_paged_multi``; the
prefill output elementwise within the contract with
``oracle.prefill_attn_paged`` (the causal score matrix per head).  Slots past
each sequence's last position hold NaN, so a read past it would show.
"""

import zlib

import numpy as np
import pytest
import torch

import oracle
from contract import assert_contract
from gpu_util import down_bits, down_f64, log, up
from workloads import make_paged_prefill

pytestmark = pytest.mark.gpu

kvd = pytest.importorskip("kv_cache_decode_02_amd")


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


class Dev:
    def __init__(self, inp):
        self.inp = inp
        self.q, self.k, self.v = up(inp.q), up(inp.k_pool), up(inp.v_pool)
        self.kn, self.vn = up(inp.k_new), up(inp.v_new)
        self.cu, self.table, self.seq = up(inp.cu_rows), up(inp.block_table), up(inp.seq_lens)

    def append(self):
        kvd.kv_append_paged_multi(self.k, self.v, self.kn, self.vn, self.cu, self.table, self.seq,
                                  self.inp.max_rows)


CASES = [
    ("prefill-r4", dict(H_q=32, H_kv=8, d=128, past=[0, 0, 0], new=[1, 37, 200])),
    ("chunked-r4", dict(H_q=32, H_kv=8, d=128, past=[17, 100, 1000, 3], new=[64, 5, 130, 1])),
    ("decode-rows", dict(H_q=32, H_kv=8, d=128, past=[15, 16, 4095], new=[1, 1, 1])),
    ("mha-d64", dict(H_q=4, H_kv=4, d=64, past=[0, 50], new=[90, 33])),
    ("r8-d128", dict(H_q=64, H_kv=8, d=128, past=[10, 500], new=[40, 70])),
    ("r2-d64", dict(H_q=8, H_kv=4, d=64, past=[31, 0], new=[17, 64])),
    ("r16-mqa", dict(H_q=16, H_kv=1, d=128, past=[7, 0], new=[9, 20])),
]


@pytest.mark.parametrize("name,c", CASES, ids=[n for n, _ in CASES])
def test_prefill_parity(name, c):
    log(f"prefill {name}")
    inp = make_paged_prefill(np.random.default_rng(zlib.crc32(name.encode())), len(c["past"]),
                             c["H_q"], c["H_kv"], c["d"], c["past"], c["new"])
    dev = Dev(inp)
    dev.append()
    out = kvd.prefill_attn_paged(dev.q, dev.k, dev.v, dev.cu, dev.table, dev.seq,
                                 inp.max_seq_len, inp.max_rows)
    torch.cuda.synchronize()
    k2, v2 = oracle.append_paged_multi(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new,
                                       inp.cu_rows, inp.block_table, inp.seq_lens)
    assert np.array_equal(down_bits(dev.k), k2) and np.array_equal(down_bits(dev.v), v2)
    ref = oracle.prefill_attn_paged(inp.q, k2, v2, inp.block_table, inp.seq_lens, inp.cu_rows,
                                    "bf16")
    rep = assert_contract(down_f64(out), ref, name)
    log(f"  max_err {rep['max_err']:.3e} scaled {rep['scaled']:.3e}")


def test_sequence_without_new_rows_is_skipped():
    log("prefill with an empty chunk")
    inp = make_paged_prefill(np.random.default_rng(3), 3, 8, 2, 128, [5, 40, 0], [3, 0, 4])
    dev = Dev(inp)
    dev.append()
    out = kvd.prefill_attn_paged(dev.q, dev.k, dev.v, dev.cu, dev.table, dev.seq,
                                 inp.max_seq_len, inp.max_rows)
    torch.cuda.synchronize()
    k2, v2 = oracle.append_paged_multi(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new,
                                       inp.cu_rows, inp.block_table, inp.seq_lens)
    ref = oracle.prefill_attn_paged(inp.q, k2, v2, inp.block_table, inp.seq_lens, inp.cu_rows,
                                    "bf16")
    assert_contract(down_f64(out), ref, "empty chunk")


def test_prefill_full_size_sampled():
    name = "prefill_llama3_8b"
    log(f"full {name}: generating")
    from workloads import make_config_inputs
    inp = make_config_inputs(name)[0]
    dev = Dev(inp)
    dev.append()
    out = kvd.prefill_attn_paged(dev.q, dev.k, dev.v, dev.cu, dev.table, dev.seq,
                                 inp.max_seq_len, inp.max_rows)
    torch.cuda.synchronize()
    got = down_f64(out)
    assert np.all(np.isfinite(got))
    k2, v2 = oracle.append_paged_multi(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new,
                                       inp.cu_rows, inp.block_table, inp.seq_lens)
    rng = np.random.default_rng(6)
    for b in range(inp.B):
        n = int(inp.cu_rows[b + 1] - inp.cu_rows[b])
        L = int(inp.seq_lens[b])
        K = oracle.to_f64(oracle.gather_logical(k2, inp.block_table, b, L), "bf16")
        V = oracle.to_f64(oracle.gather_logical(v2, inp.block_table, b, L), "bf16")
        for i in [0, n - 1, int(rng.integers(n))]:
            p = L - n + i
            row = inp.cu_rows[b] + i
            ref = oracle.decode_attention(oracle.to_f64(inp.q[row], "bf16"), K[:p + 1], V[:p + 1])
            assert_contract(got[row], ref, f"{name} b={b} row={i}")
    log(f"full {name}: ok")
