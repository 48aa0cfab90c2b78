"""ctypes binding of libkvdecode.so: argument marshalling only.

Every computation happens in the HIP library; this module turns torch tensors
into device pointers and sizes, passes torch's current HIP stream, and maps
negative status codes to exceptions (ValueError for argument errors,
RuntimeError for HIP runtime errors).  Importing it fails loudly when the
library has not been built.
"""

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvdecode.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "kvdecode.h")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python kv_cache_decode_02_amd/build.py or __graft_entry__.build())")

lib = ctypes.CDLL(LIB_PATH)

KVD_F32 = 0
KVD_BF16 = 1

_vp = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t
_f = ctypes.c_float

lib.kvd_status_string.restype = ctypes.c_char_p
lib.kvd_status_string.argtypes = [_i]
lib.kv_append_paged.restype = _i
lib.kv_append_paged.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp]
lib.decode_attn_partition_tokens.restype = _i
lib.decode_attn_partition_tokens.argtypes = [_i, _i, _i, _i, _i, _i]
lib.decode_attn_workspace_bytes.restype = _sz
lib.decode_attn_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i]
_PAGED_ARGS = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _f, _i, _vp, _sz, _i, _vp]
lib.decode_attn_paged.restype = _i
lib.decode_attn_paged.argtypes = [_vp] + _PAGED_ARGS
lib.decode_attn_paged_partials.restype = _i
lib.decode_attn_paged_partials.argtypes = _PAGED_ARGS
# q, k_cache, v_cache, k_new, v_new, then the paged arguments from block_table on
_APPEND_ARGS = _PAGED_ARGS[:3] + [_vp, _vp] + _PAGED_ARGS[3:]
lib.decode_attn_paged_append.restype = _i
lib.decode_attn_paged_append.argtypes = [_vp] + _APPEND_ARGS
lib.decode_attn_paged_append_partials.restype = _i
lib.decode_attn_paged_append_partials.argtypes = _APPEND_ARGS
lib.decode_attn_paged_append_noalloc.restype = _i
# the append arguments without the workspace pointer and byte count
lib.decode_attn_paged_append_noalloc.argtypes = [_vp] + _APPEND_ARGS[:-4] + [_i, _vp]
lib.decode_attn_noalloc_scratch_bytes.restype = _sz
lib.decode_attn_noalloc_scratch_bytes.argtypes = []
lib.kvd_stream_read_sink_bytes.restype = _sz
lib.kvd_stream_read_sink_bytes.argtypes = []
lib.kvd_stream_read.restype = _i
lib.kvd_stream_read.argtypes = [_vp, _sz, _vp, _sz, _vp]
lib.kvd_lds_read_sink_bytes.restype = _sz
lib.kvd_lds_read_sink_bytes.argtypes = [_i]
lib.kvd_lds_read_bytes.restype = ctypes.c_longlong
lib.kvd_lds_read_bytes.argtypes = [_i, _i, _i]
lib.kvd_lds_read.restype = _i
lib.kvd_lds_read.argtypes = [_i, _i, _i, _vp, _vp, _sz, _vp]
_MLA_ARGS = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _f, _i, _vp, _sz, _vp]
lib.decode_attn_mla.restype = _i
lib.decode_attn_mla.argtypes = [_vp] + _MLA_ARGS
lib.decode_attn_mla_partials.restype = _i
lib.decode_attn_mla_partials.argtypes = _MLA_ARGS
# q, c_cache, c_new, then the MLA arguments from block_table on
_MLA_APPEND_ARGS = _MLA_ARGS[:2] + [_vp] + _MLA_ARGS[2:]
lib.decode_attn_mla_append.restype = _i
lib.decode_attn_mla_append.argtypes = [_vp] + _MLA_APPEND_ARGS
lib.decode_attn_mla_append_partials.restype = _i
lib.decode_attn_mla_append_partials.argtypes = _MLA_APPEND_ARGS
lib.kv_append_paged_int8.restype = _i
lib.kv_append_paged_int8.argtypes = [_vp] * 8 + [_i] * 7 + [_vp]
# q, k_cache, v_cache, k_scale, v_scale, then the paged arguments from block_table on
_INT8_ARGS = _PAGED_ARGS[:3] + [_vp, _vp] + _PAGED_ARGS[3:]
lib.decode_attn_paged_int8.restype = _i
lib.decode_attn_paged_int8.argtypes = [_vp] + _INT8_ARGS
lib.decode_attn_paged_int8_partials.restype = _i
lib.decode_attn_paged_int8_partials.argtypes = _INT8_ARGS
lib.kv_append_paged_fp8.restype = _i
lib.kv_append_paged_fp8.argtypes = [_vp] * 8 + [_i] * 7 + [_vp]
lib.decode_attn_paged_fp8.restype = _i
lib.decode_attn_paged_fp8.argtypes = [_vp] + _INT8_ARGS
lib.decode_attn_paged_fp8_partials.restype = _i
lib.decode_attn_paged_fp8_partials.argtypes = _INT8_ARGS
# the paged arguments with `window` after `scale`
_WINDOW_ARGS = _PAGED_ARGS[:14] + [_i] + _PAGED_ARGS[14:]
lib.decode_attn_paged_window.restype = _i
lib.decode_attn_paged_window.argtypes = [_vp] + _WINDOW_ARGS
lib.decode_attn_paged_window_partials.restype = _i
lib.decode_attn_paged_window_partials.argtypes = _WINDOW_ARGS
lib.kv_copy_blocks.restype = _i
lib.kv_copy_blocks.argtypes = [_vp, _vp, _i, _sz, _i, _vp]
_i64 = ctypes.c_int64
lib.kvd_block_hashes.restype = _i
lib.kvd_block_hashes.argtypes = [_vp, _i64, _i, _vp, _sz, _vp]
lib.kvd_pool_create.restype = _vp
lib.kvd_pool_create.argtypes = [_i, _i]
lib.kvd_pool_destroy.restype = None
lib.kvd_pool_destroy.argtypes = [_vp]
for _name in ("kvd_pool_available", "kvd_pool_used", "kvd_seq_create"):
    getattr(lib, _name).restype = _i
    getattr(lib, _name).argtypes = [_vp]
lib.kvd_pool_block_ref.restype = _i
lib.kvd_pool_block_ref.argtypes = [_vp, _i]
for _name in ("kvd_seq_fork", "kvd_seq_release"):
    getattr(lib, _name).restype = _i
    getattr(lib, _name).argtypes = [_vp, _i]
lib.kvd_seq_len.restype = _i64
lib.kvd_seq_len.argtypes = [_vp, _i]
lib.kvd_seq_table.restype = _i
lib.kvd_seq_table.argtypes = [_vp, _i, _vp, _i]
lib.kvd_seq_append.restype = _i
lib.kvd_seq_append.argtypes = [_vp, _i, _i, _vp, _i, _vp]
lib.kvd_seq_commit_hashes.restype = _i
lib.kvd_seq_commit_hashes.argtypes = [_vp, _i, _vp, _i]
lib.kvd_seq_create_with_prefix.restype = _i
lib.kvd_seq_create_with_prefix.argtypes = [_vp, _vp, _i, _vp]
lib.kv_append_paged_multi.restype = _i
lib.kv_append_paged_multi.argtypes = [_vp] * 7 + [_i] * 8 + [_vp]
lib.prefill_attn_paged.restype = _i
lib.prefill_attn_paged.argtypes = [_vp] * 7 + [_i] * 9 + [_f, _i, _vp]
lib.decode_attn_merge.restype = _i
lib.decode_attn_merge.argtypes = [_vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _sz, _i, _vp]
lib.kvd_validate_tables.restype = _i
lib.kvd_validate_tables.argtypes = [_vp, _vp, _i, _i, _i, _i, _vp, _vp]
lib.kvd_validate_finite.restype = _i
lib.kvd_validate_finite.argtypes = [_vp, _sz, _i]


class KvdError(ValueError):
    """An argument was rejected by the library's host-side checks."""


def _check(status, what):
    if status == 0:
        return
    msg = f"{what}: {lib.kvd_status_string(status).decode()} (status {status})"
    if status == -5:
        raise RuntimeError(msg)
    raise KvdError(msg)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return KVD_BF16
    if t.dtype == torch.float32:
        return KVD_F32
    raise KvdError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, device=True, dtype=None, contiguous=True, like=None):
    """Device, dtype and contiguity of an argument; ``like``: a tensor whose
    device it must share."""
    if t is None:
        raise KvdError(f"{name} is required")
    if device and not t.is_cuda:
        raise KvdError(f"{name} must be a device tensor")
    if like is not None and t.device != like.device:
        raise KvdError(f"{name} must be on {like.device} (is on {t.device})")
    if dtype is not None and t.dtype != dtype:
        raise KvdError(f"{name} must be {dtype}")
    if contiguous and not t.is_contiguous():
        raise KvdError(f"{name} must be contiguous")


# Shape checks run before anything else (before the device checks too): a
# kernel indexes every argument from the sizes of the others, so a short
# seq_lens, block table or output would be read or written past its end.
def _dims(t, name, shape):
    """``t`` has len(shape) dimensions with the given sizes (None: any)."""
    if t is None:
        raise KvdError(f"{name} is required")
    if t.dim() != len(shape) or any(w is not None and int(w) != int(n)
                                    for w, n in zip(shape, t.shape)):
        want = ", ".join("*" if w is None else str(int(w)) for w in shape)
        raise KvdError(f"{name} must be [{want}], got {list(t.shape)}")


def _batch(seq_lens, block_table, B):
    """seq_lens [B] and block_table [B, max_blocks_per_seq]."""
    _dims(seq_lens, "seq_lens", (B,))
    _dims(block_table, "block_table", (B, None))


def kv_append_paged(k_cache, v_cache, k_new, v_new, block_table, seq_lens, stream=None):
    """Write each sequence's new row at position seq_lens[b] - 1 of its cache.

    k_cache/v_cache: [num_blocks, 16, H_kv, d]; k_new/v_new: [B, H_kv, d];
    v_cache and v_new may both be None (latent cache).
    """
    _dims(k_cache, "k_cache", (None,) * 4)
    nb, bs, h_kv, d = k_cache.shape
    _dims(k_new, "k_new", (None, h_kv, d))
    B = k_new.shape[0]
    _batch(seq_lens, block_table, B)
    if (v_cache is None) != (v_new is None):
        raise KvdError("v_cache and v_new must both be given or both be None")
    if v_cache is not None:
        _dims(v_cache, "v_cache", tuple(k_cache.shape))
        _dims(v_new, "v_new", tuple(k_new.shape))
    _need(k_cache, "k_cache")
    _need(k_new, "k_new", dtype=k_cache.dtype, like=k_cache)
    if v_cache is not None:
        _need(v_cache, "v_cache", dtype=k_cache.dtype, like=k_cache)
        _need(v_new, "v_new", dtype=k_cache.dtype, like=k_cache)
    _need(block_table, "block_table", dtype=torch.int32, like=k_cache)
    _need(seq_lens, "seq_lens", dtype=torch.int32, like=k_cache)
    status = lib.kv_append_paged(_ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new),
                                 _ptr(block_table), _ptr(seq_lens), B, h_kv, d, bs,
                                 block_table.shape[1], nb, _dtype_code(k_cache), _stream(stream))
    _check(status, "kv_append_paged")


def decode_attn_partition_tokens(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                 partition_tokens=0):
    r = lib.decode_attn_partition_tokens(batch, num_q_heads, num_kv_heads, head_dim,
                                         max_seq_len, partition_tokens)
    _check(min(r, 0), "decode_attn_partition_tokens")
    return r


def decode_attn_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                partition_tokens=0):
    n = lib.decode_attn_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim,
                                        max_seq_len, partition_tokens)
    if n == 0 and batch != 0:
        raise KvdError("decode_attn_workspace_bytes: invalid sizes")
    return n


def alloc_workspace(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len, partition_tokens=0,
              device="cuda"):
    """A device buffer of the size the decode calls need (torch allocation)."""
    n = decode_attn_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                    partition_tokens)
    return torch.empty(n, dtype=torch.uint8, device=device)


def _paged_args(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, scale,
                partition_tokens, ws, out=None):
    _dims(q, "q", (None,) * 3)
    B, h_q, d = q.shape
    _dims(k_cache, "k_cache", (None, None, None, d))
    _dims(v_cache, "v_cache", tuple(k_cache.shape))
    nb, bs, h_kv, _ = k_cache.shape
    _batch(seq_lens, block_table, B)
    if out is not None:
        _dims(out, "out", (B, h_q, d))
        _need(out, "out", dtype=q.dtype, like=q)
    # ws None: the allocation-free entry point, which takes no workspace
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")) + (
            () if ws is None else ((ws, "workspace"),)):
        _need(t, n, like=q)
    _need(block_table, "block_table", dtype=torch.int32, like=q)
    _need(seq_lens, "seq_lens", dtype=torch.int32, like=q)
    if q.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype:
        raise KvdError("q, k_cache and v_cache must share one dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return [_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
            B, h_q, h_kv, d, bs, block_table.shape[1], nb, int(max_seq_len), float(scale),
            int(partition_tokens), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
            _dtype_code(q)]


def decode_attn_paged(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, scale=None,
                      partition_tokens=0, workspace=None, out=None, stream=None):
    """Decode attention of q [B, H_q, d] over the paged K/V caches; returns out."""
    _dims(q, "q", (None,) * 3)
    _dims(k_cache, "k_cache", (None,) * 4)
    B, h_q, d = q.shape
    h_kv = k_cache.shape[2]
    if workspace is None:
        workspace = alloc_workspace(B, h_q, h_kv, d, max_seq_len, partition_tokens,
                                    device=q.device)
    if out is None:
        out = torch.empty_like(q)
    args = _paged_args(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, scale,
                       partition_tokens, workspace, out)
    _check(lib.decode_attn_paged(_ptr(out), *args, _stream(stream)), "decode_attn_paged")
    return out


def decode_attn_paged_partials(q, k_cache, v_cache, block_table, seq_lens, max_seq_len,
                               workspace, scale=None, partition_tokens=0, stream=None):
    """First phase only: fills ``workspace`` with per-partition partials."""
    args = _paged_args(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, scale,
                       partition_tokens, workspace)
    _check(lib.decode_attn_paged_partials(*args, _stream(stream)), "decode_attn_paged_partials")


def decode_attn_paged_window(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, window,
                             scale=None, partition_tokens=0, workspace=None, out=None,
                             stream=None):
    """decode_attn_paged under a sliding window: each row attends to its
    last ``window`` positions; returns out."""
    _dims(q, "q", (None,) * 3)
    _dims(k_cache, "k_cache", (None,) * 4)
    B, h_q, d = q.shape
    h_kv = k_cache.shape[2]
    if workspace is None:
        workspace = alloc_workspace(B, h_q, h_kv, d, max_seq_len, partition_tokens,
                                    device=q.device)
    if out is None:
        out = torch.empty_like(q)
    args = _paged_args(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, scale,
                       partition_tokens, workspace, out)
    args = args[:14] + [int(window)] + args[14:]
    _check(lib.decode_attn_paged_window(_ptr(out), *args, _stream(stream)),
           "decode_attn_paged_window")
    return out


def decode_attn_paged_window_partials(q, k_cache, v_cache, block_table, seq_lens, max_seq_len,
                                      window, workspace, scale=None, partition_tokens=0,
                                      stream=None):
    """First phase of decode_attn_paged_window; finish with decode_attn_merge."""
    args = _paged_args(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, scale,
                       partition_tokens, workspace)
    args = args[:14] + [int(window)] + args[14:]
    _check(lib.decode_attn_paged_window_partials(*args, _stream(stream)),
           "decode_attn_paged_window_partials")


def _append_args(q, k_cache, v_cache, k_new, v_new, block_table, seq_lens, max_seq_len, scale,
                 partition_tokens, ws, out=None):
    _dims(q, "q", (None,) * 3)
    _dims(k_cache, "k_cache", (None, None, None, q.shape[2]))
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _dims(t, n, (q.shape[0], k_cache.shape[2], k_cache.shape[3]))
    args = _paged_args(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, scale,
                       partition_tokens, ws, out)
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, n, dtype=k_cache.dtype, like=q)
    return args[:3] + [_ptr(k_new), _ptr(v_new)] + args[3:]


def decode_attn_paged_append(q, k_cache, v_cache, k_new, v_new, block_table, seq_lens,
                             max_seq_len, scale=None, partition_tokens=0, workspace=None,
                             out=None, stream=None):
    """kv_append_paged + decode_attn_paged in one pass: writes k_new / v_new
    [B, H_kv, d] into their slots and attends over the history plus them."""
    _dims(q, "q", (None,) * 3)
    _dims(k_cache, "k_cache", (None,) * 4)
    B, h_q, d = q.shape
    h_kv = k_cache.shape[2]
    if workspace is None:
        workspace = alloc_workspace(B, h_q, h_kv, d, max_seq_len, partition_tokens,
                                    device=q.device)
    if out is None:
        out = torch.empty_like(q)
    args = _append_args(q, k_cache, v_cache, k_new, v_new, block_table, seq_lens, max_seq_len,
                        scale, partition_tokens, workspace, out)
    _check(lib.decode_attn_paged_append(_ptr(out), *args, _stream(stream)),
           "decode_attn_paged_append")
    return out


def decode_attn_paged_append_partials(q, k_cache, v_cache, k_new, v_new, block_table, seq_lens,
                                      max_seq_len, workspace, scale=None, partition_tokens=0,
                                      stream=None):
    """First phase of decode_attn_paged_append only (the append included)."""
    args = _append_args(q, k_cache, v_cache, k_new, v_new, block_table, seq_lens, max_seq_len,
                        scale, partition_tokens, workspace)
    _check(lib.decode_attn_paged_append_partials(*args, _stream(stream)),
           "decode_attn_paged_append_partials")


def decode_attn_paged_append_noalloc(q, k_cache, v_cache, k_new, v_new, block_table, seq_lens,
                                     max_seq_len, out, scale=None, partition_tokens=0,
                                     stream=None):
    """decode_attn_paged_append without a workspace argument and without any
    device allocation: the library's per-GPU scratch array holds the partial
    results (at most decode_attn_noalloc_scratch_bytes()).  ``out`` is
    required; calls that overlap on one GPU race on the scratch array."""
    if out is None:
        raise KvdError("out is required (the allocation-free call allocates nothing)")
    args = _append_args(q, k_cache, v_cache, k_new, v_new, block_table, seq_lens, max_seq_len,
                        scale, partition_tokens, None, out)
    # the C entry point takes no workspace: drop the pointer and byte count
    del args[-3:-1]
    _check(lib.decode_attn_paged_append_noalloc(_ptr(out), *args, _stream(stream)),
           "decode_attn_paged_append_noalloc")
    return out


def decode_attn_noalloc_scratch_bytes():
    return int(lib.decode_attn_noalloc_scratch_bytes())


def stream_read(src, sink, stream=None):
    """Measurement aid: one streaming read of the device tensor ``src`` (its
    byte size a multiple of 16); ``sink`` a device tensor of at least
    stream_read_sink_bytes() bytes."""
    _need(src, "src")
    _need(sink, "sink", like=src)
    _check(lib.kvd_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                               sink.numel() * sink.element_size(), _stream(stream)),
           "kvd_stream_read")


def stream_read_sink_bytes():
    return int(lib.kvd_stream_read_sink_bytes())


def lds_read(mode, groups, iters, cycles, sink, stream=None):
    """Measurement aid: ``groups`` workgroups read their LDS ``iters`` times
    (mode 0: 16-byte reads, 1: 8-byte transposing reads).  ``cycles`` is a
    device int64 tensor of ``groups`` words (shader clock cycles of each
    workgroup's read loop); ``sink`` a device tensor of at least
    lds_read_sink_bytes(groups) bytes."""
    _need(cycles, "cycles", dtype=torch.int64)
    _need(sink, "sink", like=cycles)
    if cycles.numel() < groups:
        raise KvdError(f"kvd_lds_read: cycles holds {cycles.numel()} words, need {groups}")
    _check(lib.kvd_lds_read(int(mode), int(groups), int(iters), _ptr(cycles), _ptr(sink),
                            sink.numel() * sink.element_size(), _stream(stream)),
           "kvd_lds_read")


def lds_read_sink_bytes(groups):
    return int(lib.kvd_lds_read_sink_bytes(int(groups)))


def lds_read_bytes(mode, groups, iters):
    return int(lib.kvd_lds_read_bytes(int(mode), int(groups), int(iters)))


def decode_attn_merge(out, seq_lens, num_kv_heads, max_seq_len, workspace, partition_tokens=0,
                      stream=None):
    """Second phase only: merges the partials in ``workspace`` into ``out``."""
    _dims(out, "out", (None,) * 3)
    B, h_q, d = out.shape
    _dims(seq_lens, "seq_lens", (B,))
    _need(out, "out")
    _need(seq_lens, "seq_lens", dtype=torch.int32, like=out)
    _need(workspace, "workspace", like=out)
    status = lib.decode_attn_merge(_ptr(out), _ptr(seq_lens), B, h_q, num_kv_heads, d,
                                   int(max_seq_len), int(partition_tokens), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(),
                                   _dtype_code(out), _stream(stream))
    _check(status, "decode_attn_merge")


MLA_D_C = 512
MLA_D_ROPE = 64


def mla_default_scale(d_c=MLA_D_C, d_rope=MLA_D_ROPE):
    """1/sqrt(d_c/4 + d_rope): the un-absorbed per-head key width when d_c = 4 d_h."""
    return 1.0 / math.sqrt(d_c // 4 + d_rope)


def _mla_args(q, c_cache, block_table, seq_lens, max_seq_len, d_c, scale, partition_tokens, ws,
              out=None):
    _dims(q, "q", (None,) * 3)
    B, h, w = q.shape
    if c_cache is None or c_cache.dim() < 3:
        raise KvdError("c_cache must be [num_blocks, 16, d_c + d_rope]")
    nb, bs = c_cache.shape[0], c_cache.shape[1]
    if c_cache.shape[-1] != w or c_cache.numel() != nb * bs * w:
        raise KvdError("c_cache must be [num_blocks, 16, d_c + d_rope] like q's rows")
    _batch(seq_lens, block_table, B)
    if out is not None:
        _dims(out, "out", (B, h, d_c))
        _need(out, "out", dtype=torch.bfloat16, like=q)
    _need(q, "q", dtype=torch.bfloat16)
    _need(c_cache, "c_cache", dtype=torch.bfloat16, like=q)
    _need(ws, "workspace", like=q)
    _need(block_table, "block_table", dtype=torch.int32, like=q)
    _need(seq_lens, "seq_lens", dtype=torch.int32, like=q)
    if scale is None:
        scale = mla_default_scale(d_c, w - d_c)
    return [_ptr(q), _ptr(c_cache), _ptr(block_table), _ptr(seq_lens), B, h, d_c, w - d_c, bs,
            block_table.shape[1], nb, int(max_seq_len), float(scale), int(partition_tokens),
            _ptr(ws), ws.numel() * ws.element_size()]


def decode_attn_mla(q, c_cache, block_table, seq_lens, max_seq_len, d_c=MLA_D_C, scale=None,
                    partition_tokens=0, workspace=None, out=None, stream=None):
    """Absorbed-MLA decode of q [B, H, d_c + d_rope] over the latent cache; returns
    out [B, H, d_c] (bf16)."""
    _dims(q, "q", (None,) * 3)
    B, h, _ = q.shape
    if workspace is None:
        workspace = alloc_workspace(B, h, 1, d_c, max_seq_len, partition_tokens, device=q.device)
    if out is None:
        out = torch.empty((B, h, d_c), dtype=torch.bfloat16, device=q.device)
    args = _mla_args(q, c_cache, block_table, seq_lens, max_seq_len, d_c, scale,
                     partition_tokens, workspace, out)
    _check(lib.decode_attn_mla(_ptr(out), *args, _stream(stream)), "decode_attn_mla")
    return out


def decode_attn_mla_partials(q, c_cache, block_table, seq_lens, max_seq_len, workspace,
                             d_c=MLA_D_C, scale=None, partition_tokens=0, stream=None):
    """First phase of decode_attn_mla; finish with decode_attn_merge(out, seq_lens, 1, ...)."""
    args = _mla_args(q, c_cache, block_table, seq_lens, max_seq_len, d_c, scale,
                     partition_tokens, workspace)
    _check(lib.decode_attn_mla_partials(*args, _stream(stream)), "decode_attn_mla_partials")


def _mla_append_args(q, c_cache, c_new, block_table, seq_lens, max_seq_len, d_c, scale,
                     partition_tokens, ws, out=None):
    if c_new is None or c_new.dim() < 2 or c_new.shape[0] != q.shape[0] or \
            c_new.numel() != q.shape[0] * q.shape[2]:
        raise KvdError("c_new must be [B, d_c + d_rope] (one latent row per sequence)")
    args = _mla_args(q, c_cache, block_table, seq_lens, max_seq_len, d_c, scale,
                     partition_tokens, ws, out)
    _need(c_new, "c_new", dtype=torch.bfloat16, like=q)
    return args[:2] + [_ptr(c_new)] + args[2:]


def decode_attn_mla_append(q, c_cache, c_new, block_table, seq_lens, max_seq_len, d_c=MLA_D_C,
                           scale=None, partition_tokens=0, workspace=None, out=None,
                           stream=None):
    """kv_append_paged of c_new [B, d_c + d_rope] + decode_attn_mla in one pass:
    writes each row into its slot and attends over the history plus it."""
    _dims(q, "q", (None,) * 3)
    B, h, _ = q.shape
    if workspace is None:
        workspace = alloc_workspace(B, h, 1, d_c, max_seq_len, partition_tokens, device=q.device)
    if out is None:
        out = torch.empty((B, h, d_c), dtype=torch.bfloat16, device=q.device)
    args = _mla_append_args(q, c_cache, c_new, block_table, seq_lens, max_seq_len, d_c, scale,
                            partition_tokens, workspace, out)
    _check(lib.decode_attn_mla_append(_ptr(out), *args, _stream(stream)), "decode_attn_mla_append")
    return out


def decode_attn_mla_append_partials(q, c_cache, c_new, block_table, seq_lens, max_seq_len,
                                    workspace, d_c=MLA_D_C, scale=None, partition_tokens=0,
                                    stream=None):
    """First phase of decode_attn_mla_append only (the append included)."""
    args = _mla_append_args(q, c_cache, c_new, block_table, seq_lens, max_seq_len, d_c, scale,
                            partition_tokens, workspace)
    _check(lib.decode_attn_mla_append_partials(*args, _stream(stream)),
           "decode_attn_mla_append_partials")


# --- INT8 cache -----------------------------------------------------------------

def kv_append_paged_int8(k_cache, v_cache, v_scale, k_new, v_new, k_scale, block_table,
                         seq_lens, stream=None):
    """Quantise each sequence's new row into position seq_lens[b] - 1 of an INT8
    cache: K per channel with ``k_scale`` [H_kv, d], V per token (the scale of
    the row goes to ``v_scale`` [num_blocks, 16, H_kv]).

    k_cache/v_cache: int8 [num_blocks, 16, H_kv, d]; k_new/v_new: [B, H_kv, d]
    bf16 or fp32.
    """
    _append_bytes("kv_append_paged_int8", torch.int8, k_cache, v_cache, v_scale, k_new, v_new,
                  k_scale, block_table, seq_lens, stream)


def kv_append_paged_fp8(k_cache, v_cache, v_scale, k_new, v_new, k_scale, block_table,
                        seq_lens, stream=None):
    """As kv_append_paged_int8 for an FP8 cache: uint8 E4M3 codes, V scale
    max |v| / 448."""
    _append_bytes("kv_append_paged_fp8", torch.uint8, k_cache, v_cache, v_scale, k_new, v_new,
                  k_scale, block_table, seq_lens, stream)


def _append_bytes(name, code_dtype, k_cache, v_cache, v_scale, k_new, v_new, k_scale,
                  block_table, seq_lens, stream):
    _dims(k_cache, "k_cache", (None,) * 4)
    nb, bs, h_kv, d = k_cache.shape
    _dims(v_cache, "v_cache", tuple(k_cache.shape))
    _dims(v_scale, "v_scale", (nb, bs, h_kv))
    _dims(k_scale, "k_scale", (h_kv, d))
    _dims(k_new, "k_new", (None, h_kv, d))
    B = k_new.shape[0]
    _dims(v_new, "v_new", (B, h_kv, d))
    _batch(seq_lens, block_table, B)
    _need(k_cache, "k_cache", dtype=code_dtype)
    _need(v_cache, "v_cache", dtype=code_dtype, like=k_cache)
    _need(v_scale, "v_scale", dtype=torch.float32, like=k_cache)
    _need(k_scale, "k_scale", dtype=torch.float32, like=k_cache)
    _need(k_new, "k_new", like=k_cache)
    _need(v_new, "v_new", dtype=k_new.dtype, like=k_cache)
    _need(block_table, "block_table", dtype=torch.int32, like=k_cache)
    _need(seq_lens, "seq_lens", dtype=torch.int32, like=k_cache)
    status = getattr(lib, name)(_ptr(k_cache), _ptr(v_cache), _ptr(v_scale), _ptr(k_new),
                                _ptr(v_new), _ptr(k_scale), _ptr(block_table), _ptr(seq_lens), B,
                                h_kv, d, bs, block_table.shape[1], nb, _dtype_code(k_new),
                                _stream(stream))
    _check(status, name)


def _int8_args(q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens, max_seq_len, scale,
               partition_tokens, ws, code_dtype=torch.int8, out=None):
    _dims(q, "q", (None,) * 3)
    B, h_q, d = q.shape
    _dims(k_cache, "k_cache", (None, None, None, d))
    _dims(v_cache, "v_cache", tuple(k_cache.shape))
    nb, bs, h_kv, _ = k_cache.shape
    _dims(k_scale, "k_scale", (h_kv, d))
    _dims(v_scale, "v_scale", (nb, bs, h_kv))
    _batch(seq_lens, block_table, B)
    if out is not None:
        _dims(out, "out", (B, h_q, d))
        _need(out, "out", dtype=torch.bfloat16, like=q)
    _need(q, "q", dtype=torch.bfloat16)
    _need(ws, "workspace", like=q)
    _need(k_cache, "k_cache", dtype=code_dtype, like=q)
    _need(v_cache, "v_cache", dtype=code_dtype, like=q)
    _need(k_scale, "k_scale", dtype=torch.float32, like=q)
    _need(v_scale, "v_scale", dtype=torch.float32, like=q)
    _need(block_table, "block_table", dtype=torch.int32, like=q)
    _need(seq_lens, "seq_lens", dtype=torch.int32, like=q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return [_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
            _ptr(block_table), _ptr(seq_lens), B, h_q, h_kv, d, bs, block_table.shape[1], nb,
            int(max_seq_len), float(scale), int(partition_tokens), _ptr(ws),
            ws.numel() * ws.element_size(), KVD_BF16]


def decode_attn_paged_int8(q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens,
                           max_seq_len, scale=None, partition_tokens=0, workspace=None, out=None,
                           stream=None):
    """Decode attention of bf16 q [B, H_q, d] over an INT8 paged cache; returns
    the bf16 output."""
    _dims(q, "q", (None,) * 3)
    _dims(k_cache, "k_cache", (None,) * 4)
    B, h_q, d = q.shape
    h_kv = k_cache.shape[2]
    if workspace is None:
        workspace = alloc_workspace(B, h_q, h_kv, d, max_seq_len, partition_tokens,
                                    device=q.device)
    if out is None:
        out = torch.empty_like(q)
    args = _int8_args(q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens, max_seq_len,
                      scale, partition_tokens, workspace, out=out)
    _check(lib.decode_attn_paged_int8(_ptr(out), *args, _stream(stream)),
           "decode_attn_paged_int8")
    return out


def decode_attn_paged_int8_partials(q, k_cache, v_cache, k_scale, v_scale, block_table,
                                    seq_lens, max_seq_len, workspace, scale=None,
                                    partition_tokens=0, stream=None):
    """First phase of decode_attn_paged_int8 only; finish with decode_attn_merge."""
    args = _int8_args(q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens, max_seq_len,
                      scale, partition_tokens, workspace)
    _check(lib.decode_attn_paged_int8_partials(*args, _stream(stream)),
           "decode_attn_paged_int8_partials")


def decode_attn_paged_fp8(q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens,
                          max_seq_len, scale=None, partition_tokens=0, workspace=None, out=None,
                          stream=None):
    """Decode attention of bf16 q [B, H_q, d] over an FP8 (E4M3, uint8 codes)
    paged cache; returns the bf16 output."""
    _dims(q, "q", (None,) * 3)
    _dims(k_cache, "k_cache", (None,) * 4)
    B, h_q, d = q.shape
    h_kv = k_cache.shape[2]
    if workspace is None:
        workspace = alloc_workspace(B, h_q, h_kv, d, max_seq_len, partition_tokens,
                                    device=q.device)
    if out is None:
        out = torch.empty_like(q)
    args = _int8_args(q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens, max_seq_len,
                      scale, partition_tokens, workspace, code_dtype=torch.uint8, out=out)
    _check(lib.decode_attn_paged_fp8(_ptr(out), *args, _stream(stream)), "decode_attn_paged_fp8")
    return out


def decode_attn_paged_fp8_partials(q, k_cache, v_cache, k_scale, v_scale, block_table,
                                   seq_lens, max_seq_len, workspace, scale=None,
                                   partition_tokens=0, stream=None):
    """First phase of decode_attn_paged_fp8 only; finish with decode_attn_merge."""
    args = _int8_args(q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens, max_seq_len,
                      scale, partition_tokens, workspace, code_dtype=torch.uint8)
    _check(lib.decode_attn_paged_fp8_partials(*args, _stream(stream)),
           "decode_attn_paged_fp8_partials")


# --- block copies and the host block pool ----------------------------------------

def validate_tables(seq_lens, block_table, num_blocks, max_seq_len=0, new_rows=None):
    """The library's host-side precondition check on host int32 arrays
    (numpy or CPU tensors); returns None, raises KvdError naming the first
    offending sequence."""
    import numpy as np
    lens = np.ascontiguousarray(np.asarray(seq_lens), dtype=np.int32)
    table = np.ascontiguousarray(np.asarray(block_table), dtype=np.int32)
    if table.ndim != 2 or table.shape[0] != lens.shape[0]:
        raise KvdError("validate_tables: block_table must be [batch, max_blocks_per_seq]")
    rows = None if new_rows is None else np.ascontiguousarray(np.asarray(new_rows), dtype=np.int32)
    bad = ctypes.c_int(-1)
    st = lib.kvd_validate_tables(lens.ctypes.data, table.ctypes.data, lens.shape[0],
                                 table.shape[1], num_blocks, max_seq_len,
                                 None if rows is None else rows.ctypes.data, ctypes.byref(bad))
    if st:
        raise KvdError(f"validate_tables: {lib.kvd_status_string(st).decode()} "
                       f"(status {st}, sequence {bad.value})")


def validate_finite(values, dtype="bf16"):
    """The library's host-side finiteness check: uint16 bf16 bit patterns or
    float32 values in a host array; raises KvdError on NaN or infinity."""
    import numpy as np
    a = np.ascontiguousarray(values, dtype=np.uint16 if dtype == "bf16" else np.float32)
    code = KVD_BF16 if dtype == "bf16" else KVD_F32
    _check(lib.kvd_validate_finite(a.ctypes.data, a.size, code), "validate_finite")


def kv_copy_blocks(cache, pairs, stream=None):
    """Copy whole blocks of ``cache`` [num_blocks, ...]: block pairs[i, 0] onto
    block pairs[i, 1] (device int32 [n, 2])."""
    if pairs is None or pairs.numel() and (pairs.dim() != 2 or pairs.shape[1] != 2):
        raise KvdError("pairs must be [n, 2]")
    _need(cache, "cache")
    _need(pairs, "pairs", dtype=torch.int32, like=cache)
    n = pairs.shape[0] if pairs.numel() else 0
    nb = cache.shape[0]
    block_bytes = cache[0].numel() * cache.element_size()
    _check(lib.kv_copy_blocks(_ptr(cache), _ptr(pairs), n, block_bytes, nb, _stream(stream)),
           "kv_copy_blocks")


def block_hashes(tokens, block_size, identity=b""):
    """Chained 32-byte keys of the full blocks of a token list (host)."""
    toks = (ctypes.c_int32 * max(1, len(tokens)))(*[int(t) for t in tokens])
    full = len(tokens) // block_size if block_size > 0 else 0
    out = (ctypes.c_uint8 * max(1, 32 * full))()
    ident = ctypes.create_string_buffer(bytes(identity), max(1, len(identity)))
    r = lib.kvd_block_hashes(toks, len(tokens), block_size, ident, len(identity), out)
    _check(min(r, 0), "kvd_block_hashes")
    raw = bytes(out)
    return [raw[32 * j:32 * (j + 1)] for j in range(r)]


class PoolExhausted(KvdError):
    """The block pool has too few free blocks for the request."""


class BlockPool:
    """Host-side paged block allocator (reference counts, fork, copy-on-write,
    prefix reuse through chained block keys); see include/kvdecode.h."""

    def __init__(self, num_blocks, block_size=16):
        self._p = lib.kvd_pool_create(num_blocks, block_size)
        if not self._p:
            raise KvdError("kvd_pool_create: invalid sizes or out of memory")
        self.block_size = block_size

    def close(self):
        if self._p:
            lib.kvd_pool_destroy(self._p)
            self._p = None

    def __del__(self):
        self.close()

    def _ok(self, r, what):
        if r == -6:
            raise PoolExhausted(f"{what}: {lib.kvd_status_string(r).decode()}")
        _check(min(r, 0), what)
        return r

    def available(self):
        return self._ok(lib.kvd_pool_available(self._p), "kvd_pool_available")

    def used(self):
        return self._ok(lib.kvd_pool_used(self._p), "kvd_pool_used")

    def ref(self, block):
        return self._ok(lib.kvd_pool_block_ref(self._p, block), "kvd_pool_block_ref")

    def create(self):
        return self._ok(lib.kvd_seq_create(self._p), "kvd_seq_create")

    def fork(self, seq):
        return self._ok(lib.kvd_seq_fork(self._p, seq), "kvd_seq_fork")

    def release(self, seq):
        self._ok(lib.kvd_seq_release(self._p, seq), "kvd_seq_release")

    def length(self, seq):
        r = lib.kvd_seq_len(self._p, seq)
        self._ok(min(r, 0), "kvd_seq_len")
        return r

    def table(self, seq):
        n = self.length(seq) // self.block_size + 1
        buf = (ctypes.c_int32 * max(1, n))()
        r = self._ok(lib.kvd_seq_table(self._p, seq, buf, n), "kvd_seq_table")
        return list(buf[:r])

    def append(self, seq, num_tokens):
        """Reserve num_tokens slots; returns the (old, new) block copies to do first."""
        pairs = (ctypes.c_int32 * 2)()
        n = ctypes.c_int(0)
        self._ok(lib.kvd_seq_append(self._p, seq, num_tokens, pairs, 1, ctypes.byref(n)),
                 "kvd_seq_append")
        return [(pairs[0], pairs[1])] if n.value else []

    def commit(self, seq, keys):
        raw = b"".join(keys)
        buf = ctypes.create_string_buffer(raw, max(1, len(raw)))
        self._ok(lib.kvd_seq_commit_hashes(self._p, seq, buf, len(keys)), "kvd_seq_commit_hashes")

    def create_with_prefix(self, keys):
        raw = b"".join(keys)
        buf = ctypes.create_string_buffer(raw, max(1, len(raw)))
        hit = ctypes.c_int(0)
        s = self._ok(lib.kvd_seq_create_with_prefix(self._p, buf, len(keys), ctypes.byref(hit)),
                     "kvd_seq_create_with_prefix")
        return s, hit.value


# --- chunked prefill / multi-token decode ----------------------------------------

def kv_append_paged_multi(k_cache, v_cache, k_new, v_new, cu_rows, block_table, seq_lens,
                          max_rows, stream=None):
    """Write n_b = cu_rows[b+1] - cu_rows[b] new rows of each sequence into
    positions [seq_lens[b] - n_b, seq_lens[b]); k_new/v_new: [N, H_kv, d]."""
    _dims(k_cache, "k_cache", (None,) * 4)
    nb, bs, h_kv, d = k_cache.shape
    _dims(v_cache, "v_cache", tuple(k_cache.shape))
    _dims(k_new, "k_new", (None, h_kv, d))
    _dims(v_new, "v_new", tuple(k_new.shape))
    _dims(seq_lens, "seq_lens", (None,))
    B = seq_lens.shape[0]
    _batch(seq_lens, block_table, B)
    _dims(cu_rows, "cu_rows", (B + 1,))
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache"), (k_new, "k_new"), (v_new, "v_new")):
        _need(t, n, dtype=k_cache.dtype, like=k_cache)
    for t, n in ((cu_rows, "cu_rows"), (block_table, "block_table"), (seq_lens, "seq_lens")):
        _need(t, n, dtype=torch.int32, like=k_cache)
    status = lib.kv_append_paged_multi(_ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new),
                                       _ptr(cu_rows), _ptr(block_table), _ptr(seq_lens), B,
                                       int(max_rows), h_kv, d, bs, block_table.shape[1], nb,
                                       _dtype_code(k_cache), _stream(stream))
    _check(status, "kv_append_paged_multi")


def prefill_attn_paged(q, k_cache, v_cache, cu_rows, block_table, seq_lens, max_seq_len,
                       max_rows, scale=None, out=None, stream=None):
    """Causal attention of the new rows q [N, H_q, d] (bf16) over the paged
    cache, which already holds them; returns out [N, H_q, d]."""
    _dims(q, "q", (None,) * 3)
    N, h_q, d = q.shape
    _dims(k_cache, "k_cache", (None, None, None, d))
    _dims(v_cache, "v_cache", tuple(k_cache.shape))
    nb, bs, h_kv, _ = k_cache.shape
    _dims(seq_lens, "seq_lens", (None,))
    B = seq_lens.shape[0]
    _batch(seq_lens, block_table, B)
    _dims(cu_rows, "cu_rows", (B + 1,))
    if out is None:
        out = torch.empty_like(q)
    _dims(out, "out", (N, h_q, d))
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (out, "out")):
        _need(t, n, dtype=torch.bfloat16, like=q)
    for t, n in ((cu_rows, "cu_rows"), (block_table, "block_table"), (seq_lens, "seq_lens")):
        _need(t, n, dtype=torch.int32, like=q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    status = lib.prefill_attn_paged(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                    _ptr(cu_rows), _ptr(block_table), _ptr(seq_lens), B,
                                    int(max_rows), h_q, h_kv, d, bs, block_table.shape[1], nb,
                                    int(max_seq_len), float(scale), KVD_BF16, _stream(stream))
    _check(status, "prefill_attn_paged")
    return out
