"""Seeded generators for paged decode inputs (no attention arithmetic here).

Layout produced (the library's documented layout):
  q        [B, H_q, d]
  k_pool   [NB, block_size, H_kv, d]    physical blocks, token-major inside
  v_pool   [NB, block_size, H_kv, d]
  k_new    [B, H_kv, d]                 this step's token, not yet in the pool
  v_new    [B, H_kv, d]
  block_table int32 [B, MB]             unused entries hold UNUSED_TABLE_ENTRY
  seq_lens    int32 [B]                 length after this step's append

Storage: 'bf16' arrays are uint16 bit patterns (fp32 draws rounded to nearest
even); 'f32' arrays are float32.

Physical placement: the pool has exactly sum ceil(seq_lens / block_size)
blocks.  One seeded permutation of the pool is handed out in order, request by
request, logical block by logical block (``table='permuted'``), or the blocks
are handed out in pool order (``table='identity'``, the contiguous cache).

Slots that hold no cached history -- this step's slot, which the append will
fill, and the unused tail of each request's last block -- are filled with a
sentinel: NaN in parity runs (an over-read or a missing append shows up as a
NaN output) or zero in timing runs.

Draw order from the generator (fixed): block permutation, q, K pool, V pool,
k_new, v_new.  Sequence lengths are drawn by the caller before this.

INT8 caches (``make_paged_decode_int8``) hold codes in [-127, 127] drawn
uniformly, per-channel K scales [H_kv, d] and per-token V scales
[NB, block_size, H_kv] drawn uniformly in std * [0.5, 1.5] / 64, so that the
cached values have roughly the spread of the bf16 workloads; k_new / v_new are
bf16 draws (the append quantises them).  Unfilled slots hold code -128 (never
written by the append) and a NaN V scale in parity runs, code 0 and scale 0
in timing runs.  Draw order: block permutation, q, K codes, V codes, V
scales, K scales, k_new, v_new.

FP8 caches (``make_paged_decode_fp8``) hold E4M3 bytes: a uniform sign and a
magnitude code uniform in 0x00 .. 0x3F (the values 0 .. 1.875, from 2^-9 up
through the subnormals and eight binades), K and V scales uniform in
std * [0.5, 1.5], so that the cached values again have roughly the spread of
the bf16 workloads.  With ``full_range`` the magnitude codes cover every
finite value 0x00 .. 0x7E (up to 448) and the scales are std * [0.5, 1.5] / 256.  Unfilled slots hold code 0x7F (E4M3 NaN, never written
by the append) and a NaN V scale in parity runs, code 0 and scale 0 in timing
runs.  Same draw order as the INT8 caches.
"""

from dataclasses import dataclass

import numpy as np

BLOCK_SIZE = 16
UNUSED_TABLE_ENTRY = np.int32(2**31 - 1)
BF16_NAN = np.uint16(0x7FC0)
_CHUNK = 1 << 22  # values drawn per generator call (fixed: keeps streams stable)


def bf16_round_bits(x):
    """float32 array -> bf16 bit patterns (uint16), round to nearest even.

    Inputs must be finite.  The low 16 bits are dropped after adding
    0x7FFF plus the lowest kept bit, which rounds ties to even.
    """
    a = np.ascontiguousarray(x, dtype=np.float32)
    u = a.view(np.uint32)
    keep_lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + keep_lsb) >> np.uint32(16)).astype(np.uint16)


def _draw(rng, shape, std, dtype):
    """Normal(0, std^2) values of ``shape`` in storage ``dtype``, chunked."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)
    for start in range(0, n, _CHUNK):
        stop = min(start + _CHUNK, n)
        v = rng.standard_normal(stop - start, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        out[start:stop] = bf16_round_bits(v) if dtype == "bf16" else v
    return out.reshape(shape)


def _sentinel(dtype, kind):
    if kind == "nan":
        return BF16_NAN if dtype == "bf16" else np.float32(np.nan)
    if kind == "zero":
        return np.uint16(0) if dtype == "bf16" else np.float32(0)
    raise ValueError(f"unknown sentinel {kind!r}")


def _blocks_needed(length, block_size):
    return -(-int(length) // block_size)


def _assign_blocks(rng, seq_lens, block_size, max_blocks, table):
    """Build the block table; return (table, num_blocks, per-request block lists)."""
    counts = [_blocks_needed(n, block_size) for n in seq_lens]
    nb = int(sum(counts))
    if table == "permuted":
        order = rng.permutation(nb).astype(np.int32)
    elif table == "identity":
        order = np.arange(nb, dtype=np.int32)
    else:
        raise ValueError(f"unknown table kind {table!r}")
    bt = np.full((len(seq_lens), max_blocks), UNUSED_TABLE_ENTRY, dtype=np.int32)
    owned = []
    pos = 0
    for b, c in enumerate(counts):
        if c > max_blocks:
            raise ValueError("max_blocks_per_seq too small for the lengths")
        bt[b, :c] = order[pos:pos + c]
        owned.append(order[pos:pos + c])
        pos += c
    return bt, nb, owned


def _mark_unfilled(pool, owned, seq_lens, block_size, value):
    """Put ``value`` in every slot of a request's last block past its history.

    Request b has seq_lens[b] - 1 history rows; its blocks were handed out in
    order, so the last block it owns holds the final history rows followed by
    the slot reserved for this step's token and the unused tail.
    """
    for blocks, n in zip(owned, seq_lens):
        hist = int(n) - 1
        last = int(blocks[-1])
        filled_in_last = hist - (len(blocks) - 1) * block_size
        pool[last, filled_in_last:] = value


@dataclass
class PagedDecodeInputs:
    dtype: str
    B: int
    H_q: int
    H_kv: int
    d: int
    block_size: int
    seq_lens: np.ndarray
    block_table: np.ndarray
    num_blocks: int
    q: np.ndarray
    k_pool: np.ndarray
    v_pool: np.ndarray
    k_new: np.ndarray
    v_new: np.ndarray

    @property
    def max_blocks_per_seq(self):
        return int(self.block_table.shape[1])

    @property
    def max_seq_len(self):
        return int(self.seq_lens.max())

    @property
    def kv_bytes_read(self):
        """K and V bytes of all visible positions (what one decode call reads)."""
        elem = 2 if self.dtype == "bf16" else 4
        return int(2 * int(self.seq_lens.astype(np.int64).sum()) * self.H_kv * self.d * elem)


def make_paged_decode(rng, B, H_q, H_kv, d, seq_lens, dtype="bf16", table="permuted",
                      std=1.0, sentinel="nan", max_blocks_per_seq=None,
                      block_size=BLOCK_SIZE):
    """Draw one decode step's inputs; see the module docstring for the layout."""
    lens = np.asarray(seq_lens, dtype=np.int64)
    if lens.shape != (B,):
        raise ValueError("seq_lens must have B entries")
    if np.any(lens < 1):
        raise ValueError("every sequence holds at least the appended token")
    if H_q % H_kv != 0:
        raise ValueError("H_q must be a multiple of H_kv")
    mb = max_blocks_per_seq or _blocks_needed(lens.max(), block_size)
    bt, nb, owned = _assign_blocks(rng, lens, block_size, mb, table)
    q = _draw(rng, (B, H_q, d), std, dtype)
    k_pool = _draw(rng, (nb, block_size, H_kv, d), std, dtype)
    v_pool = _draw(rng, (nb, block_size, H_kv, d), std, dtype)
    k_new = _draw(rng, (B, H_kv, d), std, dtype)
    v_new = _draw(rng, (B, H_kv, d), std, dtype)
    if sentinel is not None:
        val = _sentinel(dtype, sentinel)
        _mark_unfilled(k_pool, owned, lens, block_size, val)
        _mark_unfilled(v_pool, owned, lens, block_size, val)
    return PagedDecodeInputs(dtype, B, H_q, H_kv, d, block_size, lens.astype(np.int32),
                             bt, nb, q, k_pool, v_pool, k_new, v_new)


@dataclass
class MlaInputs:
    B: int
    H: int
    d_c: int
    d_rope: int
    block_size: int
    seq_lens: np.ndarray
    block_table: np.ndarray
    num_blocks: int
    q: np.ndarray       # [B, H, d_c + d_rope] bf16 bits (absorbed queries)
    c_pool: np.ndarray  # [NB, block_size, d_c + d_rope] bf16 bits
    c_new: np.ndarray   # [B, d_c + d_rope] bf16 bits
    dtype: str = "bf16"

    @property
    def width(self):
        return self.d_c + self.d_rope

    @property
    def max_blocks_per_seq(self):
        return int(self.block_table.shape[1])

    @property
    def max_seq_len(self):
        return int(self.seq_lens.max())

    @property
    def kv_bytes_read(self):
        return int(int(self.seq_lens.astype(np.int64).sum()) * self.width * 2)


def make_mla(rng, B, H, d_c, d_rope, seq_lens, std, table="permuted", sentinel="nan",
             max_blocks_per_seq=None, block_size=BLOCK_SIZE):
    """Draw one absorbed-MLA decode step's inputs (bf16 storage).

    Draw order: block permutation, q, latent pool, new latent rows.
    """
    lens = np.asarray(seq_lens, dtype=np.int64)
    if lens.shape != (B,) or np.any(lens < 1):
        raise ValueError("seq_lens must have B entries, each >= 1")
    w = d_c + d_rope
    mb = max_blocks_per_seq or _blocks_needed(lens.max(), block_size)
    bt, nb, owned = _assign_blocks(rng, lens, block_size, mb, table)
    q = _draw(rng, (B, H, w), std, "bf16")
    c_pool = _draw(rng, (nb, block_size, w), std, "bf16")
    c_new = _draw(rng, (B, w), std, "bf16")
    if sentinel is not None:
        _mark_unfilled(c_pool, owned, lens, block_size, _sentinel("bf16", sentinel))
    return MlaInputs(B, H, d_c, d_rope, block_size, lens.astype(np.int32), bt, nb,
                     q, c_pool, c_new)


def _codes(rng, shape):
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.int8)
    for start in range(0, n, _CHUNK):
        stop = min(start + _CHUNK, n)
        out[start:stop] = rng.integers(-127, 128, size=stop - start, dtype=np.int8)
    return out.reshape(shape)


def _scales(rng, shape, std):
    v = rng.random(int(np.prod(shape)), dtype=np.float32) + np.float32(0.5)
    return (v * np.float32(std / 64.0)).reshape(shape)


@dataclass
class PagedInt8Inputs:
    B: int
    H_q: int
    H_kv: int
    d: int
    block_size: int
    seq_lens: np.ndarray
    block_table: np.ndarray
    num_blocks: int
    q: np.ndarray        # bf16 bits [B, H_q, d]
    kq_pool: np.ndarray  # int8 [NB, 16, H_kv, d]
    vq_pool: np.ndarray  # int8 [NB, 16, H_kv, d]
    vs_pool: np.ndarray  # fp32 [NB, 16, H_kv]
    k_scale: np.ndarray  # fp32 [H_kv, d]
    k_new: np.ndarray    # bf16 bits [B, H_kv, d]
    v_new: np.ndarray    # bf16 bits [B, H_kv, d]
    dtype: str = "bf16"  # of q, k_new, v_new and the output
    codes: str = "int8"  # "int8" codes, or "fp8": uint8 E4M3 bytes

    @property
    def max_blocks_per_seq(self):
        return int(self.block_table.shape[1])

    @property
    def max_seq_len(self):
        return int(self.seq_lens.max())

    @property
    def kv_bytes_read(self):
        """Codes of K and V plus the V scales of all visible positions."""
        n = int(self.seq_lens.astype(np.int64).sum())
        return int(n * self.H_kv * (2 * self.d + 4))


def make_paged_decode_int8(rng, B, H_q, H_kv, d, seq_lens, table="permuted", std=1.0,
                           sentinel="nan", max_blocks_per_seq=None, block_size=BLOCK_SIZE):
    """Draw one decode step's inputs over an INT8 cache (see the module docstring)."""
    lens = np.asarray(seq_lens, dtype=np.int64)
    if lens.shape != (B,) or np.any(lens < 1):
        raise ValueError("seq_lens must have B entries, each >= 1")
    if H_q % H_kv != 0:
        raise ValueError("H_q must be a multiple of H_kv")
    mb = max_blocks_per_seq or _blocks_needed(lens.max(), block_size)
    bt, nb, owned = _assign_blocks(rng, lens, block_size, mb, table)
    q = _draw(rng, (B, H_q, d), std, "bf16")
    kq = _codes(rng, (nb, block_size, H_kv, d))
    vq = _codes(rng, (nb, block_size, H_kv, d))
    vs = _scales(rng, (nb, block_size, H_kv), std)
    ks = _scales(rng, (H_kv, d), std)
    k_new = _draw(rng, (B, H_kv, d), std, "bf16")
    v_new = _draw(rng, (B, H_kv, d), std, "bf16")
    if sentinel == "nan":
        code, scale = np.int8(-128), np.float32(np.nan)
    elif sentinel == "zero":
        code, scale = np.int8(0), np.float32(0)
    else:
        raise ValueError(f"unknown sentinel {sentinel!r}")
    _mark_unfilled(kq, owned, lens, block_size, code)
    _mark_unfilled(vq, owned, lens, block_size, code)
    _mark_unfilled(vs, owned, lens, block_size, scale)
    return PagedInt8Inputs(B, H_q, H_kv, d, block_size, lens.astype(np.int32), bt, nb, q, kq, vq,
                           vs, ks, k_new, v_new)


def _fp8_codes(rng, shape, full_range=False):
    """E4M3 bytes with a uniform sign bit.  Magnitude codes uniform in
    0x00 .. 0x3F, or with ``full_range`` in 0x00 .. 0x7E (every finite
    magnitude, up to 448; 0x7F is NaN and is never drawn)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint8)
    for start in range(0, n, _CHUNK):
        stop = min(start + _CHUNK, n)
        if full_range:
            v = rng.integers(0, 254, size=stop - start, dtype=np.int32)
            out[start:stop] = ((v % 127) | ((v // 127) << 7)).astype(np.uint8)
        else:
            v = rng.integers(0, 256, size=stop - start, dtype=np.int32).astype(np.uint8)
            out[start:stop] = v & np.uint8(0xBF)  # bit 7 sign, bit 6 cleared
    return out.reshape(shape)


def make_paged_decode_fp8(rng, B, H_q, H_kv, d, seq_lens, table="permuted", std=1.0,
                          sentinel="nan", max_blocks_per_seq=None, block_size=BLOCK_SIZE,
                          full_range=False):
    """Draw one decode step's inputs over an FP8 (E4M3) cache (see the module
    docstring).  ``full_range``: history codes over every finite magnitude
    (0x00 .. 0x7E) with scales std * [0.5, 1.5] / 256."""
    lens = np.asarray(seq_lens, dtype=np.int64)
    if lens.shape != (B,) or np.any(lens < 1):
        raise ValueError("seq_lens must have B entries, each >= 1")
    if H_q % H_kv != 0:
        raise ValueError("H_q must be a multiple of H_kv")
    mb = max_blocks_per_seq or _blocks_needed(lens.max(), block_size)
    bt, nb, owned = _assign_blocks(rng, lens, block_size, mb, table)
    q = _draw(rng, (B, H_q, d), std, "bf16")
    kq = _fp8_codes(rng, (nb, block_size, H_kv, d), full_range)
    vq = _fp8_codes(rng, (nb, block_size, H_kv, d), full_range)
    sstd = std / 4.0 if full_range else std * 64.0
    vs = _scales(rng, (nb, block_size, H_kv), sstd)
    ks = _scales(rng, (H_kv, d), sstd)
    k_new = _draw(rng, (B, H_kv, d), std, "bf16")
    v_new = _draw(rng, (B, H_kv, d), std, "bf16")
    if sentinel == "nan":
        code, scale = np.uint8(0x7F), np.float32(np.nan)
    elif sentinel == "zero":
        code, scale = np.uint8(0), np.float32(0)
    else:
        raise ValueError(f"unknown sentinel {sentinel!r}")
    _mark_unfilled(kq, owned, lens, block_size, code)
    _mark_unfilled(vq, owned, lens, block_size, code)
    _mark_unfilled(vs, owned, lens, block_size, scale)
    return PagedInt8Inputs(B, H_q, H_kv, d, block_size, lens.astype(np.int32), bt, nb, q, kq, vq,
                           vs, ks, k_new, v_new, codes="fp8")


@dataclass
class PagedPrefillInputs:
    dtype: str
    B: int
    H_q: int
    H_kv: int
    d: int
    block_size: int
    seq_lens: np.ndarray     # int32 [B]: history + new rows
    cu_rows: np.ndarray      # int32 [B + 1]: new rows of sequence b are cu[b] .. cu[b+1]-1
    block_table: np.ndarray
    num_blocks: int
    q: np.ndarray            # [N, H_q, d]
    k_pool: np.ndarray       # [NB, 16, H_kv, d], history filled
    v_pool: np.ndarray
    k_new: np.ndarray        # [N, H_kv, d]
    v_new: np.ndarray

    @property
    def max_blocks_per_seq(self):
        return int(self.block_table.shape[1])

    @property
    def max_seq_len(self):
        return int(self.seq_lens.max())

    @property
    def max_rows(self):
        return int(np.max(np.diff(self.cu_rows))) if self.B else 0

    @property
    def num_rows(self):
        return int(self.cu_rows[-1])


def make_paged_prefill(rng, B, H_q, H_kv, d, past_lens, new_lens, dtype="bf16",
                       table="permuted", std=1.0, sentinel="nan", block_size=BLOCK_SIZE):
    """Chunked prefill / multi-token decode inputs: sequence b holds past_lens[b]
    cached rows and appends new_lens[b] rows this call (queries for each).
    Draw order: block permutation, q, K pool, V pool, k_new, v_new.  Slots of
    the new rows and the unused tail hold the sentinel."""
    past = np.asarray(past_lens, dtype=np.int64)
    new = np.asarray(new_lens, dtype=np.int64)
    if past.shape != (B,) or new.shape != (B,) or np.any(past < 0) or np.any(new < 0):
        raise ValueError("past_lens and new_lens must have B non-negative entries")
    lens = past + new
    if np.any(lens < 1):
        raise ValueError("every sequence needs at least one position")
    if H_q % H_kv != 0:
        raise ValueError("H_q must be a multiple of H_kv")
    mb = _blocks_needed(lens.max(), block_size)
    bt, nb, owned = _assign_blocks(rng, lens, block_size, mb, table)
    N = int(new.sum())
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(new)
    q = _draw(rng, (N, H_q, d), std, dtype)
    k_pool = _draw(rng, (nb, block_size, H_kv, d), std, dtype)
    v_pool = _draw(rng, (nb, block_size, H_kv, d), std, dtype)
    k_new = _draw(rng, (N, H_kv, d), std, dtype)
    v_new = _draw(rng, (N, H_kv, d), std, dtype)
    if sentinel is not None:
        val = _sentinel(dtype, sentinel)
        for blocks, p in zip(owned, past):
            # every slot from position p on is unfilled
            for j, blk in enumerate(blocks):
                start = max(0, int(p) - j * block_size)
                if start < block_size:
                    k_pool[int(blk), start:] = val
                    v_pool[int(blk), start:] = val
    return PagedPrefillInputs(dtype, B, H_q, H_kv, d, block_size, lens.astype(np.int32), cu, bt,
                              nb, q, k_pool, v_pool, k_new, v_new)
