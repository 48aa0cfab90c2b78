// Host-side checks of the preconditions that the kernels take on trust: the
// lengths, the block-table entries a call reads, the exclusive ownership of
// the blocks it writes, and finite small inputs.  kvd_validate_tables and
// kvd_validate_finite work on host arrays; with the environment variable
// KVD_VALIDATE=1 every entry point copies its seq_lens, block table and query
// / new rows to the host first (synchronising its stream) and refuses the
// call with KVD_ERR_SHAPE when a check fails.  The kernels themselves treat a
// length <= 0 as empty and skip table entries outside the pool; these checks
// exist to find the caller's mistake, not to make the kernels safe.
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <unordered_map>
#include <vector>

#include "../../include/kvdecode.h"
#include "kvd_internal.h"
#include "kvd_validate.h"

namespace kvd {

namespace {

constexpr int kBlock = 16;
// Pools up to this many blocks are counted in a flat array, larger ones in a
// hash map (the table entries actually used are few in comparison).
constexpr long long kFlatCountLimit = 1LL << 24;

bool finite_bits(const void* data, size_t count, int dtype) {
  if (dtype == KVD_BF16) {
    const uint16_t* h = static_cast<const uint16_t*>(data);
    for (size_t i = 0; i < count; ++i)
      if ((h[i] & 0x7F80u) == 0x7F80u) return false;
    return true;
  }
  const uint32_t* w = static_cast<const uint32_t*>(data);
  for (size_t i = 0; i < count; ++i)
    if ((w[i] & 0x7F800000u) == 0x7F800000u) return false;
  return true;
}

}  // namespace

int validate_tables(const int32_t* seq_lens, const int32_t* block_table, int batch,
                    int max_blocks_per_seq, int num_blocks, int max_seq_len,
                    const int32_t* new_rows, int* first_bad) {
  if (first_bad) *first_bad = -1;
  if (batch < 0 || max_blocks_per_seq < 1 || num_blocks < 1) return KVD_ERR_SHAPE;
  if (batch == 0) return KVD_OK;
  if (!seq_lens || !block_table) return KVD_ERR_NULL;
  const long long cap = static_cast<long long>(max_blocks_per_seq) * kBlock;
  const long long limit = max_seq_len > 0 && max_seq_len < cap ? max_seq_len : cap;
  auto fail = [&](int b) {
    if (first_bad) *first_bad = b;
    return KVD_ERR_SHAPE;
  };
  // Lengths, and every entry of a block holding a visible position.
  for (int b = 0; b < batch; ++b) {
    const long long len = seq_lens[b];
    if (len < 1 || len > limit) return fail(b);
    if (new_rows && (new_rows[b] < 0 || new_rows[b] > len)) return fail(b);
    const int32_t* row = block_table + static_cast<size_t>(b) * max_blocks_per_seq;
    const long long nb = (len + kBlock - 1) / kBlock;
    for (long long j = 0; j < nb; ++j)
      if (row[j] < 0 || row[j] >= num_blocks) return fail(b);
  }
  if (!new_rows) return KVD_OK;
  // A block that receives new rows must be referenced by no other sequence
  // and by no other logical block of its own sequence.
  std::vector<int32_t> flat;
  std::unordered_map<int32_t, int32_t> sparse;
  const bool use_flat = num_blocks <= kFlatCountLimit;
  if (use_flat) flat.assign(static_cast<size_t>(num_blocks), 0);
  auto count = [&](int32_t blk) -> int32_t& { return use_flat ? flat[blk] : sparse[blk]; };
  for (int b = 0; b < batch; ++b) {
    const int32_t* row = block_table + static_cast<size_t>(b) * max_blocks_per_seq;
    const long long nb = (static_cast<long long>(seq_lens[b]) + kBlock - 1) / kBlock;
    for (long long j = 0; j < nb; ++j) ++count(row[j]);
  }
  for (int b = 0; b < batch; ++b) {
    if (new_rows[b] == 0) continue;
    const int32_t* row = block_table + static_cast<size_t>(b) * max_blocks_per_seq;
    const long long first = (static_cast<long long>(seq_lens[b]) - new_rows[b]) / kBlock;
    const long long last = (static_cast<long long>(seq_lens[b]) - 1) / kBlock;
    for (long long j = first; j <= last; ++j)
      if (count(row[j]) != 1) return fail(b);
  }
  return KVD_OK;
}

int validate_finite(const void* data, size_t count, int dtype) {
  if (count == 0) return KVD_OK;
  if (!data) return KVD_ERR_NULL;
  if (dtype != KVD_BF16 && dtype != KVD_F32) return KVD_ERR_UNSUPPORTED;
  return finite_bits(data, count, dtype) ? KVD_OK : KVD_ERR_SHAPE;
}

bool validation_enabled() {
  const char* v = getenv("KVD_VALIDATE");
  return v != nullptr && strcmp(v, "1") == 0;
}

int validate_device(const DeviceChecks& c, hipStream_t stream) {
  if (c.batch == 0) return KVD_OK;
  std::vector<int32_t> lens(static_cast<size_t>(c.batch));
  std::vector<int32_t> table(static_cast<size_t>(c.batch) * c.max_blocks_per_seq);
  std::vector<int32_t> rows;
  auto copy = [&](void* dst, const void* src, size_t bytes) {
    return hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToHost, stream);
  };
  if (copy(lens.data(), c.seq_lens, lens.size() * 4) != hipSuccess ||
      copy(table.data(), c.block_table, table.size() * 4) != hipSuccess)
    return KVD_ERR_HIP;
  if (c.cu_rows) {
    rows.resize(static_cast<size_t>(c.batch) + 1);
    if (copy(rows.data(), c.cu_rows, rows.size() * 4) != hipSuccess) return KVD_ERR_HIP;
  }
  std::vector<std::vector<uint8_t>> small(c.num_finite);
  for (int i = 0; i < c.num_finite; ++i) {
    small[i].resize(c.finite[i].bytes);
    if (c.finite[i].bytes && copy(small[i].data(), c.finite[i].ptr, c.finite[i].bytes) != hipSuccess)
      return KVD_ERR_HIP;
  }
  if (hipStreamSynchronize(stream) != hipSuccess) return KVD_ERR_HIP;
  std::vector<int32_t> new_rows;
  if (c.cu_rows) {
    new_rows.resize(static_cast<size_t>(c.batch));
    for (int b = 0; b < c.batch; ++b) {
      new_rows[b] = rows[b + 1] - rows[b];
      if (new_rows[b] < 0) return KVD_ERR_SHAPE;
    }
  } else if (c.writes_last) {
    new_rows.assign(static_cast<size_t>(c.batch), 1);
  }
  int rc = validate_tables(lens.data(), table.data(), c.batch, c.max_blocks_per_seq, c.num_blocks,
                           c.max_seq_len, new_rows.empty() ? nullptr : new_rows.data(), nullptr);
  if (rc) return rc;
  for (int i = 0; i < c.num_finite; ++i) {
    const size_t elem = c.finite[i].dtype == KVD_BF16 ? 2 : 4;
    rc = validate_finite(small[i].data(), c.finite[i].bytes / elem, c.finite[i].dtype);
    if (rc) return rc;
  }
  return KVD_OK;
}

}  // namespace kvd

extern "C" {

int kvd_validate_tables(const int32_t* seq_lens, const int32_t* block_table, int batch,
                        int max_blocks_per_seq, int num_blocks, int max_seq_len,
                        const int32_t* new_rows, int* first_bad) {
  return kvd::validate_tables(seq_lens, block_table, batch, max_blocks_per_seq, num_blocks,
                              max_seq_len, new_rows, first_bad);
}

int kvd_validate_finite(const void* data, size_t count, kvd_dtype_t dtype) {
  return kvd::validate_finite(data, count, dtype);
}

}  // extern "C"
