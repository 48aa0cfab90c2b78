"""The C-ABI library: exports and host-side argument checks (CPU only).

No call here launches a kernel: each either is pure host arithmetic
(workspace sizing, partition choice) or is rejected by the host-side checks,
which run before any HIP call.
"""

import ctypes
import re

import pytest

import kv_cache_decode_02_amd as kvd
from kv_cache_decode_02_amd._native import lib

OK, ENULL, ESHAPE, EUNSUP, EWS = 0, -1, -2, -3, -4


def declared_functions():
    text = open(kvd.HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"sizeof"})


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert "kv_append_paged" in names and "decode_attn_paged" in names
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5, 7):
        assert lib.kvd_status_string(s)


def test_workspace_layout():
    # P = ceil(max_len / pt) partitions; D fp32 values and (m, l) per
    # (b, h, p), each section padded to 256 B.
    B, Hq, Hkv, D, L, pt = 3, 8, 2, 128, 1000, 256
    P = -(-L // pt)
    o = B * Hq * P * D * 4
    ml = B * Hq * P * 2 * 4
    pad = lambda x: -(-x // 256) * 256  # noqa: E731
    assert kvd.decode_attn_workspace_bytes(B, Hq, Hkv, D, L, pt) == pad(o) + pad(ml)


def test_balanced_workspace_layout():
    # Automatic mode of the paged path: at most ceil(ceil(L / 16) / 16) + 1
    # pieces per (b, h), then an int32 piece count per (b, h), each section
    # padded to 256 B.
    B, Hq, Hkv, D, L = 3, 8, 2, 128, 1000
    P = -(-(-(-L // 16)) // 16) + 1
    pad = lambda x: -(-x // 256) * 256  # noqa: E731
    want = pad(B * Hq * P * D * 4) + pad(B * Hq * P * 2 * 4) + pad(B * Hq * 4)
    assert kvd.decode_attn_workspace_bytes(B, Hq, Hkv, D, L, 0) == want


def test_partition_choice():
    assert kvd.decode_attn_partition_tokens(4, 64, 8, 128, 131072, 512) == 512
    # 0 = balanced split for the paged path
    assert kvd.decode_attn_partition_tokens(64, 32, 8, 128, 8192, 0) == 0
    assert kvd.decode_attn_partition_tokens(1, 4, 4, 32, 129, 0) == 0
    # the latent (MLA) path keeps fixed partitions: one workgroup per CU
    assert kvd.decode_attn_partition_tokens(32, 128, 1, 512, 4096, 0) == 1024
    assert kvd.decode_attn_partition_tokens(1, 128, 1, 512, 4096, 0) == 64
    # batches beyond the balanced split's limit fall back to fixed partitions
    auto = kvd.decode_attn_partition_tokens(20000, 32, 8, 128, 1024, 0)
    assert auto % 16 == 0 and 64 <= auto <= 1024
    with pytest.raises(kvd.KvdError):
        kvd.decode_attn_partition_tokens(1, 4, 4, 32, 129, 24)
    with pytest.raises(kvd.KvdError):
        kvd.decode_attn_partition_tokens(1, 4, 4, 32, 129, 2048)
    with pytest.raises(kvd.KvdError):
        kvd.decode_attn_partition_tokens(1, 6, 4, 32, 129, 0)


P = ctypes.c_void_p(0x1000)  # never dereferenced: every call below is rejected first


def append(**kw):
    a = dict(k=P, v=P, kn=P, vn=P, bt=P, sl=P, B=2, hkv=8, d=128, bs=16, mb=4, nb=8, dt=1)
    a.update(kw)
    return lib.kv_append_paged(a["k"], a["v"], a["kn"], a["vn"], a["bt"], a["sl"], a["B"],
                               a["hkv"], a["d"], a["bs"], a["mb"], a["nb"], a["dt"], None)


def test_append_rejections():
    assert append(k=None) == ENULL
    assert append(v=None) == ENULL           # v_cache without v_new
    assert append(bt=None) == ENULL
    assert append(bs=32) == EUNSUP
    assert append(dt=7) == EUNSUP
    assert append(hkv=0) == ESHAPE
    assert append(B=-1) == ESHAPE
    assert append(mb=0) == ESHAPE
    assert append(hkv=1, d=3, dt=1) == ESHAPE
    assert append(B=0) == OK                 # empty batch: nothing to do


def paged(**kw):
    a = dict(o=P, q=P, k=P, v=P, bt=P, sl=P, B=2, hq=32, hkv=8, d=128, bs=16, mb=64, nb=128,
             L=1024, scale=0.088, pt=0, ws=P, wsb=1 << 40, dt=1)
    a.update(kw)
    return lib.decode_attn_paged(a["o"], a["q"], a["k"], a["v"], a["bt"], a["sl"], a["B"],
                                 a["hq"], a["hkv"], a["d"], a["bs"], a["mb"], a["nb"], a["L"],
                                 a["scale"], a["pt"], a["ws"], a["wsb"], a["dt"], None)


def test_decode_rejections():
    assert paged(q=None) == ENULL
    assert paged(o=None) == ENULL
    assert paged(v=None) == ENULL
    assert paged(hq=30) == ESHAPE            # not a multiple of H_kv
    assert paged(hq=24) == EUNSUP            # ratio 3 not built
    assert paged(d=96) == EUNSUP
    assert paged(bs=8) == EUNSUP
    assert paged(dt=2) == EUNSUP
    assert paged(L=64 * 16 + 1) == ESHAPE    # beyond the table row
    assert paged(L=0) == ESHAPE
    assert paged(pt=40) == ESHAPE
    assert paged(ws=None) == EWS
    need = kvd.decode_attn_workspace_bytes(2, 32, 8, 128, 1024, 0)
    assert paged(wsb=need - 1) == EWS
    assert paged(B=0, ws=None, wsb=0) == OK  # empty batch: nothing to do


def test_merge_rejections():
    f = lib.decode_attn_merge
    assert f(None, P, 2, 32, 8, 128, 1024, 0, P, 1 << 40, 1, None) == ENULL
    assert f(P, P, 2, 32, 8, 96, 1024, 0, P, 1 << 40, 1, None) == EUNSUP
    assert f(P, P, 2, 32, 8, 128, 1024, 0, P, 16, 1, None) == EWS


def mla(**kw):
    a = dict(o=P, q=P, c=P, bt=P, sl=P, B=2, h=128, dc=512, dr=64, bs=16, mb=256, nb=512,
             L=4096, scale=0.07, pt=0, ws=P, wsb=1 << 40)
    a.update(kw)
    return lib.decode_attn_mla(a["o"], a["q"], a["c"], a["bt"], a["sl"], a["B"], a["h"], a["dc"],
                               a["dr"], a["bs"], a["mb"], a["nb"], a["L"], a["scale"], a["pt"],
                               a["ws"], a["wsb"], None)


def test_mla_rejections():
    assert mla(q=None) == ENULL
    assert mla(o=None) == ENULL
    assert mla(c=None) == ENULL
    assert mla(dc=256) == EUNSUP
    assert mla(dr=32) == EUNSUP
    assert mla(h=24) == EUNSUP            # not a multiple of 16
    assert mla(pt=48) == ESHAPE           # partitions are whole 32-token tiles
    assert mla(bs=32) == EUNSUP
    assert mla(L=256 * 16 + 1) == ESHAPE
    assert mla(ws=None) == EWS
    need = kvd.decode_attn_workspace_bytes(2, 128, 1, 512, 4096, 0)
    assert mla(wsb=need - 1) == EWS
    assert mla(B=0, q=None, o=None, ws=None, wsb=0) == OK


def fused(**kw):
    a = dict(o=P, q=P, k=P, v=P, kn=P, vn=P, bt=P, sl=P, B=2, hq=32, hkv=8, d=128, bs=16, mb=64,
             nb=128, L=1024, scale=0.088, pt=0, ws=P, wsb=1 << 40, dt=1)
    a.update(kw)
    return lib.decode_attn_paged_append(a["o"], a["q"], a["k"], a["v"], a["kn"], a["vn"], a["bt"],
                                        a["sl"], a["B"], a["hq"], a["hkv"], a["d"], a["bs"],
                                        a["mb"], a["nb"], a["L"], a["scale"], a["pt"], a["ws"],
                                        a["wsb"], a["dt"], None)


def test_fused_append_rejections():
    assert fused(kn=None) == ENULL
    assert fused(vn=None) == ENULL
    assert fused(o=None) == ENULL
    assert fused(q=None) == ENULL
    assert fused(kn=ctypes.c_void_p(0x1008)) == ESHAPE   # k_new not 16-byte aligned
    assert fused(hq=24) == EUNSUP
    assert fused(ws=None) == EWS
    assert fused(B=0, o=None, kn=None, vn=None, ws=None, wsb=0) == OK


def append_int8(**kw):
    a = dict(k=P, v=P, vs=P, kn=P, vn=P, ks=P, bt=P, sl=P, B=2, hkv=8, d=128, bs=16, mb=4, nb=8,
             dt=1)
    a.update(kw)
    return lib.kv_append_paged_int8(a["k"], a["v"], a["vs"], a["kn"], a["vn"], a["ks"], a["bt"],
                                    a["sl"], a["B"], a["hkv"], a["d"], a["bs"], a["mb"], a["nb"],
                                    a["dt"], None)


def test_append_int8_rejections():
    assert append_int8(vs=None) == ENULL
    assert append_int8(ks=None) == ENULL
    assert append_int8(v=None) == ENULL
    assert append_int8(d=96) == EUNSUP
    assert append_int8(bs=32) == EUNSUP
    assert append_int8(dt=7) == EUNSUP
    assert append_int8(hkv=0) == ESHAPE
    assert append_int8(mb=0) == ESHAPE
    assert append_int8(B=0, k=None, v=None, vs=None, kn=None, vn=None, ks=None) == OK


def paged_int8(**kw):
    a = dict(o=P, q=P, k=P, v=P, ks=P, vs=P, bt=P, sl=P, B=2, hq=32, hkv=8, d=128, bs=16, mb=64,
             nb=128, L=1024, scale=0.088, pt=0, ws=P, wsb=1 << 40, dt=1)
    a.update(kw)
    return lib.decode_attn_paged_int8(a["o"], a["q"], a["k"], a["v"], a["ks"], a["vs"], a["bt"],
                                      a["sl"], a["B"], a["hq"], a["hkv"], a["d"], a["bs"], a["mb"],
                                      a["nb"], a["L"], a["scale"], a["pt"], a["ws"], a["wsb"],
                                      a["dt"], None)


def test_decode_int8_rejections():
    assert paged_int8(dt=0) == EUNSUP                    # queries must be bf16
    assert paged_int8(ks=None) == ENULL
    assert paged_int8(vs=None) == ENULL
    assert paged_int8(o=None) == ENULL
    assert paged_int8(ks=ctypes.c_void_p(0x1004)) == ESHAPE  # k_scale not 16-byte aligned
    assert paged_int8(vs=ctypes.c_void_p(0x1002)) == ESHAPE  # v_scale not 4-byte aligned
    assert paged_int8(hq=24) == EUNSUP
    assert paged_int8(d=96) == EUNSUP
    assert paged_int8(ws=None) == EWS
    assert paged_int8(B=0, o=None, ks=None, vs=None, ws=None, wsb=0) == OK


def test_window_rejections():
    f = lib.decode_attn_paged_window
    args = [P, P, P, P, P, P, 2, 32, 8, 128, 16, 64, 128, 1024, 0.088]
    tail = [0, P, 1 << 40, 1, None]
    assert f(*args, 0, *tail) == ESHAPE      # window must be >= 1
    assert f(*args, -5, *tail) == ESHAPE
    assert f(*args[:1], None, *args[2:], 16, *tail) == ENULL
    assert f(*args[:6], 0, *args[7:], 16, *tail) == OK  # empty batch
