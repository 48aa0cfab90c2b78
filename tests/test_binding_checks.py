"""The Python binding rejects inconsistent sizes before any launch (CPU only).

Every kernel indexes its arguments from the sizes of the others (B from q or
k_new, the heads and head size from the cache), so a short seq_lens, block
table, output or new-row tensor would be read or written past its end on the
device.  The binding checks shapes first, then device, dtype and contiguity.
These tests use host tensors: a consistent argument set gets as far as the
device check ("must be a device tensor"), and each inconsistent one is
refused with a message that names the offending argument.  No library
function that launches work is reached.
"""

import pytest
import torch

import kv_cache_decode_02_amd as kvd
from kv_cache_decode_02_amd import KvdError

B, HQ, HKV, D, NB, MB = 3, 8, 2, 64, 10, 4
bf = torch.bfloat16
i32 = torch.int32


def paged(**over):
    a = dict(q=torch.zeros(B, HQ, D, dtype=bf), k_cache=torch.zeros(NB, 16, HKV, D, dtype=bf),
             v_cache=torch.zeros(NB, 16, HKV, D, dtype=bf),
             block_table=torch.zeros(B, MB, dtype=i32), seq_lens=torch.ones(B, dtype=i32),
             max_seq_len=64)
    a.update(over)
    return a


def ws():
    return torch.zeros(1 << 20, dtype=torch.uint8)


def new_rows(**over):
    a = dict(k_new=torch.zeros(B, HKV, D, dtype=bf), v_new=torch.zeros(B, HKV, D, dtype=bf))
    a.update(over)
    return a


BAD_BATCH = [
    ("seq_lens", dict(seq_lens=torch.ones(B - 1, dtype=i32))),
    ("seq_lens", dict(seq_lens=torch.ones(B, 1, dtype=i32))),
    ("block_table", dict(block_table=torch.zeros(B - 1, MB, dtype=i32))),
    ("block_table", dict(block_table=torch.zeros(B * MB, dtype=i32))),
]


def _refused(fn, name, *args, **kw):
    with pytest.raises(KvdError, match=name):
        fn(*args, **kw)


def _reaches_device_check(fn, *args, **kw):
    with pytest.raises(KvdError, match="device tensor"):
        fn(*args, **kw)


PAGED_FNS = [
    ("decode_attn_paged", lambda a, **k: kvd.decode_attn_paged(**a, **k)),
    ("decode_attn_paged_partials", lambda a, **k: kvd.decode_attn_paged_partials(
        **{x: y for x, y in a.items()}, workspace=ws())),
    ("decode_attn_paged_window", lambda a, **k: kvd.decode_attn_paged_window(**a, window=16, **k)),
    ("decode_attn_paged_window_partials", lambda a, **k: kvd.decode_attn_paged_window_partials(
        **a, window=16, workspace=ws())),
    ("decode_attn_paged_append", lambda a, **k: kvd.decode_attn_paged_append(
        **a, **new_rows(**{x: y for x, y in k.items() if x in ("k_new", "v_new")}),
        **{x: y for x, y in k.items() if x not in ("k_new", "v_new")})),
    ("decode_attn_paged_append_partials", lambda a, **k: kvd.decode_attn_paged_append_partials(
        **a, **new_rows(**k), workspace=ws())),
]


@pytest.mark.parametrize("fname,fn", PAGED_FNS, ids=[f[0] for f in PAGED_FNS])
def test_paged_entry_points(fname, fn):
    _reaches_device_check(fn, paged())
    for name, over in BAD_BATCH:
        _refused(fn, name, paged(**over))
    _refused(fn, "v_cache", paged(v_cache=torch.zeros(NB, 16, HKV + 1, D, dtype=bf)))
    _refused(fn, "k_cache", paged(k_cache=torch.zeros(NB, 16, HKV, D // 2, dtype=bf)))
    _refused(fn, "q", paged(q=torch.zeros(B, HQ * D, dtype=bf)))


@pytest.mark.parametrize("fname", ["decode_attn_paged", "decode_attn_paged_window",
                                   "decode_attn_paged_append"])
def test_paged_output_shape(fname):
    fn = dict(PAGED_FNS)[fname]
    _refused(fn, "out", paged(), out=torch.zeros(B, HQ, D - 1, dtype=bf))
    _refused(fn, "out", paged(), out=torch.zeros(B - 1, HQ, D, dtype=bf))


@pytest.mark.parametrize("fname", ["decode_attn_paged_append", "decode_attn_paged_append_partials"])
def test_new_rows_shape(fname):
    fn = dict(PAGED_FNS)[fname]
    _refused(fn, "k_new", paged(), k_new=torch.zeros(B - 1, HKV, D, dtype=bf))
    _refused(fn, "v_new", paged(), v_new=torch.zeros(B, HKV, D + 2, dtype=bf))


def test_merge():
    out = torch.zeros(B, HQ, D, dtype=bf)
    _reaches_device_check(kvd.decode_attn_merge, out, torch.ones(B, dtype=i32), HKV, 64, ws())
    _refused(kvd.decode_attn_merge, "seq_lens", out, torch.ones(B + 1, dtype=i32), HKV, 64, ws())
    _refused(kvd.decode_attn_merge, "out", out[0], torch.ones(B, dtype=i32), HKV, 64, ws())


def test_append():
    k = torch.zeros(NB, 16, HKV, D, dtype=bf)
    args = lambda **o: dict(dict(k_cache=k, v_cache=k.clone(), **new_rows(),  # noqa: E731
                                 block_table=torch.zeros(B, MB, dtype=i32),
                                 seq_lens=torch.ones(B, dtype=i32)), **o)
    _reaches_device_check(kvd.kv_append_paged, **args())
    for name, over in BAD_BATCH:
        _refused(kvd.kv_append_paged, name, **args(**over))
    _refused(kvd.kv_append_paged, "v_new", **args(v_new=torch.zeros(B + 1, HKV, D, dtype=bf)))
    _refused(kvd.kv_append_paged, "v_cache", **args(v_cache=torch.zeros(NB - 1, 16, HKV, D, dtype=bf)))
    _refused(kvd.kv_append_paged, "k_new", **args(k_new=torch.zeros(B, HKV, 2 * D, dtype=bf)))
    _refused(kvd.kv_append_paged, "both", **args(v_new=None))
    # latent cache: no V at all is fine up to the device check
    _reaches_device_check(kvd.kv_append_paged, **args(v_cache=None, v_new=None))


def mla(**over):
    w = 576
    a = dict(q=torch.zeros(B, 16, w, dtype=bf), c_cache=torch.zeros(NB, 16, w, dtype=bf),
             block_table=torch.zeros(B, MB, dtype=i32), seq_lens=torch.ones(B, dtype=i32),
             max_seq_len=64)
    a.update(over)
    return a


MLA_FNS = [
    ("decode_attn_mla", lambda a, **k: kvd.decode_attn_mla(**a, **k)),
    ("decode_attn_mla_partials", lambda a, **k: kvd.decode_attn_mla_partials(**a, workspace=ws())),
    ("decode_attn_mla_append", lambda a, **k: kvd.decode_attn_mla_append(
        **a, c_new=k.pop("c_new", torch.zeros(B, 576, dtype=bf)), **k)),
    ("decode_attn_mla_append_partials", lambda a, **k: kvd.decode_attn_mla_append_partials(
        **a, c_new=k.pop("c_new", torch.zeros(B, 576, dtype=bf)), workspace=ws())),
]


@pytest.mark.parametrize("fname,fn", MLA_FNS, ids=[f[0] for f in MLA_FNS])
def test_mla_entry_points(fname, fn):
    _reaches_device_check(fn, mla())
    for name, over in BAD_BATCH:
        _refused(fn, name, mla(**over))
    _refused(fn, "c_cache", mla(c_cache=torch.zeros(NB, 16, 512, dtype=bf)))
    if "append" in fname:
        _refused(fn, "c_new", mla(), c_new=torch.zeros(B - 1, 576, dtype=bf))
    if "partials" not in fname:
        _refused(fn, "out", mla(), out=torch.zeros(B, 16, 576, dtype=bf))


def one_byte(code, **over):
    a = dict(q=torch.zeros(B, HQ, D, dtype=bf), k_cache=torch.zeros(NB, 16, HKV, D, dtype=code),
             v_cache=torch.zeros(NB, 16, HKV, D, dtype=code),
             k_scale=torch.ones(HKV, D), v_scale=torch.ones(NB, 16, HKV),
             block_table=torch.zeros(B, MB, dtype=i32), seq_lens=torch.ones(B, dtype=i32),
             max_seq_len=64)
    a.update(over)
    return a


@pytest.mark.parametrize("kind,code", [("int8", torch.int8), ("fp8", torch.uint8)])
def test_one_byte_decode(kind, code):
    for fn in (getattr(kvd, f"decode_attn_paged_{kind}"),
               lambda **a: getattr(kvd, f"decode_attn_paged_{kind}_partials")(**a, workspace=ws())):
        _reaches_device_check(fn, **one_byte(code))
        for name, over in BAD_BATCH:
            _refused(fn, name, **one_byte(code, **over))
        _refused(fn, "v_scale", **one_byte(code, v_scale=torch.ones(NB, 16, HKV + 1)))
        _refused(fn, "k_scale", **one_byte(code, k_scale=torch.ones(HKV, D - 1)))
    _refused(getattr(kvd, f"decode_attn_paged_{kind}"), "out", **one_byte(code),
             out=torch.zeros(B, HQ + 1, D, dtype=bf))


@pytest.mark.parametrize("kind,code", [("int8", torch.int8), ("fp8", torch.uint8)])
def test_one_byte_append(kind, code):
    fn = getattr(kvd, f"kv_append_paged_{kind}")
    k = torch.zeros(NB, 16, HKV, D, dtype=code)
    args = lambda **o: dict(dict(k_cache=k, v_cache=k.clone(), v_scale=torch.ones(NB, 16, HKV),  # noqa: E731
                                 **new_rows(), k_scale=torch.ones(HKV, D),
                                 block_table=torch.zeros(B, MB, dtype=i32),
                                 seq_lens=torch.ones(B, dtype=i32)), **o)
    _reaches_device_check(fn, **args())
    for name, over in BAD_BATCH:
        _refused(fn, name, **args(**over))
    _refused(fn, "v_new", **args(v_new=torch.zeros(B - 1, HKV, D, dtype=bf)))
    _refused(fn, "v_scale", **args(v_scale=torch.ones(NB, 16)))


def test_multi_append_and_prefill():
    N = 7
    k = torch.zeros(NB, 16, HKV, D, dtype=bf)
    base = dict(cu_rows=torch.zeros(B + 1, dtype=i32), block_table=torch.zeros(B, MB, dtype=i32),
                seq_lens=torch.ones(B, dtype=i32))
    app = lambda **o: dict(dict(k_cache=k, v_cache=k.clone(),  # noqa: E731
                                k_new=torch.zeros(N, HKV, D, dtype=bf),
                                v_new=torch.zeros(N, HKV, D, dtype=bf), max_rows=4, **base), **o)
    _reaches_device_check(kvd.kv_append_paged_multi, **app())
    _refused(kvd.kv_append_paged_multi, "cu_rows", **app(cu_rows=torch.zeros(B, dtype=i32)))
    _refused(kvd.kv_append_paged_multi, "block_table",
             **app(block_table=torch.zeros(B + 1, MB, dtype=i32)))
    _refused(kvd.kv_append_paged_multi, "v_new", **app(v_new=torch.zeros(N - 1, HKV, D, dtype=bf)))
    pre = lambda **o: dict(dict(q=torch.zeros(N, HQ, D, dtype=bf), k_cache=k,  # noqa: E731
                                v_cache=k.clone(), max_seq_len=64, max_rows=4, **base), **o)
    _reaches_device_check(kvd.prefill_attn_paged, **pre())
    _refused(kvd.prefill_attn_paged, "cu_rows", **pre(cu_rows=torch.zeros(B + 2, dtype=i32)))
    _refused(kvd.prefill_attn_paged, "seq_lens",
             **pre(seq_lens=torch.ones(B, 1, dtype=i32)))
    _refused(kvd.prefill_attn_paged, "out", **pre(out=torch.zeros(N, HQ, D + 1, dtype=bf)))


def test_copy_blocks():
    cache = torch.zeros(NB, 16, HKV, D, dtype=bf)
    _reaches_device_check(kvd.kv_copy_blocks, cache, torch.zeros(2, 2, dtype=i32))
    _refused(kvd.kv_copy_blocks, "pairs", cache, torch.zeros(2, 3, dtype=i32))
    _refused(kvd.kv_copy_blocks, "pairs", cache, torch.zeros(4, dtype=i32))


def test_noalloc_entry_point():
    fn = kvd.decode_attn_paged_append_noalloc
    out = torch.zeros(B, HQ, D, dtype=bf)
    _reaches_device_check(fn, **paged(), **new_rows(), out=out)
    _refused(fn, "out", **paged(), **new_rows(), out=None)
    _refused(fn, "out", **paged(), **new_rows(), out=torch.zeros(B, HQ, D + 1, dtype=bf))
    for name, over in BAD_BATCH:
        _refused(fn, name, **paged(**over), **new_rows(), out=out)
    _refused(fn, "k_new", **paged(), **new_rows(k_new=torch.zeros(B + 1, HKV, D, dtype=bf)),
             out=out)
