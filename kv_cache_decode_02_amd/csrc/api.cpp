// C ABI of the decode library: host-side argument checks, partition choice
// and kernel dispatch.  Every check below runs before any HIP call, reads no
// device memory and allocates nothing; with KVD_VALIDATE=1 the entry points
// that launch kernels first also run the host-side precondition checks of
// validate.cpp, which copy seq_lens, the block table and the small inputs to
// the host (and so synchronise the stream).
#include <limits.h>
#include <stdint.h>

#include <initializer_list>

#include "../../include/kvdecode.h"
#include "kvd_internal.h"
#include "kvd_probe.h"
#include "kvd_validate.h"

namespace kvd {

namespace {

constexpr int kBlockSize = 16;
constexpr int kMinPartition = 64;
constexpr int kMaxPartition = 1024;   // 64 blocks: one block id per lane
constexpr long long kTargetWaves = 12288;
constexpr long long kMlaTargetGroups = 256;  // one workgroup per compute unit
constexpr int kLatentWidth = 512;
constexpr int kMaxBalancedBatch = 8191;  // two prefixes and the lengths in LDS (96 KiB)
constexpr int kMaxTableBlocks = 1 << 26;  // keeps max_blocks_per_seq * 16 in int

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

int heads_per_wave(int ratio) { return ratio < 4 ? ratio : 4; }

bool dtype_ok(int dtype) { return dtype == KVD_F32 || dtype == KVD_BF16; }

int elem_bytes(int dtype) { return dtype == KVD_BF16 ? 2 : 4; }

int check_heads(int batch, int num_q_heads, int num_kv_heads) {
  if (batch < 0 || num_q_heads < 1 || num_kv_heads < 1) return KVD_ERR_SHAPE;
  if (num_q_heads % num_kv_heads != 0) return KVD_ERR_SHAPE;
  return KVD_OK;
}

// Partition size: the given one, or the largest of 1024 .. 64 that still
// fills the chip for a batch at max_seq_len: kTargetWaves wavefronts for the
// paged kernel, one 512-thread workgroup per compute unit for the latent
// (MLA) kernel, whose rows are the only ones of width 512.
int resolve_partition(int batch, int num_q_heads, int num_kv_heads, int head_dim, int max_seq_len,
                      int partition_tokens) {
  if (partition_tokens > 0) {
    if (partition_tokens % kBlockSize != 0 || partition_tokens > kMaxPartition) return KVD_ERR_SHAPE;
    return partition_tokens;
  }
  if (partition_tokens < 0) return KVD_ERR_SHAPE;
  const int ratio = num_q_heads / num_kv_heads;
  const bool latent = head_dim == kLatentWidth;
  const long long units =
      latent ? static_cast<long long>(batch) * mla_head_groups(num_q_heads)
             : static_cast<long long>(batch) * num_kv_heads * (ratio / heads_per_wave(ratio));
  const long long target = latent ? kMlaTargetGroups : kTargetWaves;
  int pt = kMaxPartition;
  while (pt > kMinPartition) {
    const long long parts = (max_seq_len + pt - 1) / pt;
    if (units * parts >= target) break;
    pt /= 2;
  }
  return pt;
}

struct Sizes {
  int pt;         // 0: balanced split
  int parts;      // partitions, or the bound on pieces per sequence
  bool balanced;
  WorkspaceLayout ws;
};

int plan(int batch, int num_q_heads, int num_kv_heads, int head_dim, int max_seq_len,
         int partition_tokens, Sizes* s) {
  int rc = check_heads(batch, num_q_heads, num_kv_heads);
  if (rc) return rc;
  if (head_dim < 1 || max_seq_len < 1) return KVD_ERR_SHAPE;
  // Automatic choice for the paged path: the balanced split, unless the
  // batch is too large for its per-workgroup block prefix or its item count
  // would leave int range.
  const long long max_blocks = (max_seq_len + kBlockSize - 1) / kBlockSize;
  s->balanced = partition_tokens == 0 && head_dim != kLatentWidth && batch <= kMaxBalancedBatch &&
                static_cast<long long>(batch) * num_q_heads * max_blocks < INT_MAX;
  if (s->balanced) {
    s->pt = 0;
    s->parts = static_cast<int>((max_blocks + kBalancedMinPieceBlocks - 1) / kBalancedMinPieceBlocks) + 1;
  } else {
    const int pt = resolve_partition(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                                     partition_tokens);
    if (pt < 0) return pt;
    s->pt = pt;
    s->parts = (max_seq_len + pt - 1) / pt;
  }
  // The grid and the workspace must stay addressable.
  const long long ratio = num_q_heads / num_kv_heads;
  const long long waves = static_cast<long long>(batch) * s->parts * num_kv_heads *
                          (ratio / heads_per_wave(static_cast<int>(ratio)));
  if (waves >= INT_MAX || static_cast<long long>(batch) * num_q_heads >= INT_MAX / 4)
    return KVD_ERR_SHAPE;
  s->ws = workspace_layout(batch, num_q_heads, s->parts, head_dim, s->balanced);
  return KVD_OK;
}

int check_table(int block_size, int max_blocks_per_seq, int num_blocks, int max_seq_len) {
  if (block_size != kBlockSize) return KVD_ERR_UNSUPPORTED;
  if (max_blocks_per_seq < 1 || max_blocks_per_seq > kMaxTableBlocks || num_blocks < 1)
    return KVD_ERR_SHAPE;
  if (max_seq_len < 1 || max_seq_len > max_blocks_per_seq * kBlockSize) return KVD_ERR_SHAPE;
  return KVD_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? KVD_OK : KVD_ERR_HIP; }

// KVD_VALIDATE=1: the precondition checks of validate.cpp on this call's
// device arrays; KVD_OK without touching the device otherwise.
int preconditions(const int32_t* seq_lens, const int32_t* block_table, const int32_t* cu_rows,
                  int batch, int max_blocks_per_seq, int num_blocks, int max_seq_len,
                  bool writes_last, std::initializer_list<FiniteCheck> finite, void* stream) {
  if (!validation_enabled()) return KVD_OK;
  DeviceChecks c;
  c.seq_lens = seq_lens;
  c.block_table = block_table;
  c.cu_rows = cu_rows;
  c.batch = batch;
  c.max_blocks_per_seq = max_blocks_per_seq;
  c.num_blocks = num_blocks;
  c.max_seq_len = max_seq_len;
  c.writes_last = writes_last;
  c.num_finite = 0;
  for (const FiniteCheck& f : finite)
    if (c.num_finite < 3 && f.ptr) c.finite[c.num_finite++] = f;
  return validate_device(c, static_cast<hipStream_t>(stream));
}

size_t bytes_of(long long a, long long b, long long c, int dtype) {
  return static_cast<size_t>(a * b * c * elem_bytes(dtype));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

WorkspaceLayout workspace_layout(int batch, int num_q_heads, int num_partitions, int head_dim,
                                 bool balanced) {
  WorkspaceLayout w;
  const size_t slots = static_cast<size_t>(batch) * num_q_heads * num_partitions;
  // The latent (MLA) path stores its rows normalised, in fp16.
  w.o_bytes = slots * head_dim * (head_dim == kLatentWidth ? sizeof(uint16_t) : sizeof(float));
  w.ml_offset = align256(w.o_bytes);
  w.counts_offset = w.ml_offset + align256(slots * 2 * sizeof(float));
  const size_t counts = balanced ? static_cast<size_t>(batch) * num_q_heads * sizeof(int32_t) : 0;
  w.total = w.counts_offset + align256(counts);
  return w;
}

}  // namespace kvd

using namespace kvd;

extern "C" {

const char* kvd_status_string(int status) {
  switch (status) {
    case KVD_OK: return "ok";
    case KVD_ERR_NULL: return "a required pointer is NULL";
    case KVD_ERR_SHAPE: return "sizes are inconsistent or out of range";
    case KVD_ERR_UNSUPPORTED: return "unsupported dtype, head_dim, block_size or head ratio";
    case KVD_ERR_WORKSPACE: return "workspace is NULL or too small";
    case KVD_ERR_HIP: return "HIP runtime error";
    case KVD_ERR_NOMEM: return "block pool exhausted or host allocation failed";
    default: return "unknown status";
  }
}

int kv_append_paged(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                    const int32_t* block_table, const int32_t* seq_lens,
                    int batch, int num_kv_heads, int head_dim, int block_size,
                    int max_blocks_per_seq, int num_blocks, kvd_dtype_t dtype, void* stream) {
  if (!dtype_ok(dtype)) return KVD_ERR_UNSUPPORTED;
  if (batch < 0 || num_kv_heads < 1 || head_dim < 1 || head_dim > 1024) return KVD_ERR_SHAPE;
  if (block_size != kBlockSize) return KVD_ERR_UNSUPPORTED;
  if (max_blocks_per_seq < 1 || max_blocks_per_seq > kMaxTableBlocks || num_blocks < 1)
    return KVD_ERR_SHAPE;
  const long long row_bytes = static_cast<long long>(num_kv_heads) * head_dim * elem_bytes(dtype);
  if (row_bytes % 4 != 0 || row_bytes / 4 > INT_MAX) return KVD_ERR_SHAPE;
  if (batch == 0) return KVD_OK;  // empty batch: nothing to write, pointers unused
  if (!k_cache || !k_new || !block_table || !seq_lens) return KVD_ERR_NULL;
  if ((v_cache == nullptr) != (v_new == nullptr)) return KVD_ERR_NULL;

  AppendLaunch a;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_new = k_new;
  a.v_new = v_new;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.batch = batch;
  a.row_words = static_cast<int>(row_bytes / 4);
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.vec16 = aligned16(k_cache) && aligned16(k_new) &&
            (!v_cache || (aligned16(v_cache) && aligned16(v_new)));
  const size_t nb = static_cast<size_t>(batch) * static_cast<size_t>(row_bytes);
  const int rc = preconditions(seq_lens, block_table, nullptr, batch, max_blocks_per_seq,
                               num_blocks, 0, true, {{k_new, nb, dtype}, {v_new, nb, dtype}},
                               stream);
  if (rc) return rc;
  return hip_status(launch_append(a, static_cast<hipStream_t>(stream)));
}

int decode_attn_partition_tokens(int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                 int max_seq_len, int partition_tokens) {
  Sizes s;
  const int rc = plan(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len, partition_tokens, &s);
  return rc ? rc : s.pt;
}

size_t decode_attn_workspace_bytes(int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                   int max_seq_len, int partition_tokens) {
  Sizes s;
  if (plan(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len, partition_tokens, &s))
    return 0;
  return s.ws.total;
}

static int check_paged(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_table, const int32_t* seq_lens,
                       int batch, int num_q_heads, int num_kv_heads, int head_dim,
                       int block_size, int max_blocks_per_seq, int num_blocks,
                       int max_seq_len, int partition_tokens, const void* workspace,
                       size_t workspace_bytes, int dtype, Sizes* s) {
  if (!dtype_ok(dtype)) return KVD_ERR_UNSUPPORTED;
  int rc = check_heads(batch, num_q_heads, num_kv_heads);
  if (rc) return rc;
  if (!paged_supported(head_dim, num_q_heads / num_kv_heads, dtype == KVD_BF16))
    return KVD_ERR_UNSUPPORTED;
  rc = check_table(block_size, max_blocks_per_seq, num_blocks, max_seq_len);
  if (rc) return rc;
  rc = plan(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len, partition_tokens, s);
  if (rc) return rc;
  if (batch == 0) return KVD_OK;  // empty batch: nothing to compute, pointers unused
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens) return KVD_ERR_NULL;
  if (!workspace || workspace_bytes < s->ws.total) return KVD_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return KVD_ERR_SHAPE;
  return KVD_OK;
}

static PagedLaunch paged_launch(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_table, const int32_t* seq_lens,
                                int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                int max_blocks_per_seq, int num_blocks, int max_seq_len,
                                float scale, void* workspace, int dtype, const Sizes& s) {
  PagedLaunch a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.ws_o = static_cast<float*>(workspace);
  a.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + s.ws.ml_offset);
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.max_seq_len = max_seq_len;
  a.partition_tokens = s.pt;
  a.num_partitions = s.parts;
  a.scale = scale;
  a.bf16 = dtype == KVD_BF16;
  a.counts = s.balanced
                 ? reinterpret_cast<int*>(static_cast<char*>(workspace) + s.ws.counts_offset)
                 : nullptr;
  a.k_new = nullptr;
  a.v_new = nullptr;
  a.int8 = false;
  a.fp8 = false;
  a.k_scale = nullptr;
  a.v_scale = nullptr;
  a.window = 0;
  return a;
}

static MergeLaunch merge_launch(void* out, const int32_t* seq_lens, int batch, int num_q_heads,
                                int head_dim, int max_seq_len, const void* workspace, int dtype,
                                const Sizes& s) {
  MergeLaunch m;
  m.out = out;
  m.seq_lens = seq_lens;
  m.ws_o = static_cast<const float*>(workspace);
  m.ws_ml = reinterpret_cast<const float*>(static_cast<const char*>(workspace) + s.ws.ml_offset);
  m.batch = batch;
  m.num_q_heads = num_q_heads;
  m.head_dim = head_dim;
  m.max_blocks_per_seq_tokens = max_seq_len;
  m.partition_tokens = s.pt;
  m.num_partitions = s.parts;
  m.bf16 = dtype == KVD_BF16;
  m.counts = s.balanced ? reinterpret_cast<const int*>(static_cast<const char*>(workspace) +
                                                       s.ws.counts_offset)
                        : nullptr;
  return m;
}

int decode_attn_paged_partials(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, const int32_t* seq_lens,
                               int batch, int num_q_heads, int num_kv_heads, int head_dim,
                               int block_size, int max_blocks_per_seq, int num_blocks,
                               int max_seq_len, float scale, int partition_tokens,
                               void* workspace, size_t workspace_bytes, kvd_dtype_t dtype,
                               void* stream) {
  Sizes s;
  const int rc = check_paged(q, k_cache, v_cache, block_table, seq_lens, batch, num_q_heads,
                             num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                             max_seq_len, partition_tokens, workspace, workspace_bytes, dtype, &s);
  if (rc) return rc;
  if (batch == 0) return KVD_OK;
  const int vc = preconditions(seq_lens, block_table, nullptr, batch, max_blocks_per_seq,
                               num_blocks, max_seq_len, false,
                               {{q, bytes_of(batch, num_q_heads, head_dim, dtype), dtype}}, stream);
  if (vc) return vc;
  const PagedLaunch a = paged_launch(q, k_cache, v_cache, block_table, seq_lens, batch,
                                     num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                                     num_blocks, max_seq_len, scale, workspace, dtype, s);
  return hip_status(launch_paged_partials(a, static_cast<hipStream_t>(stream)));
}

int decode_attn_merge(void* out, const int32_t* seq_lens, int batch, int num_q_heads,
                      int num_kv_heads, int head_dim, int max_seq_len, int partition_tokens,
                      const void* workspace, size_t workspace_bytes, kvd_dtype_t dtype,
                      void* stream) {
  if (!dtype_ok(dtype)) return KVD_ERR_UNSUPPORTED;
  if (!(head_dim == 32 || head_dim == 64 || head_dim == 128 || head_dim == 512))
    return KVD_ERR_UNSUPPORTED;
  Sizes s;
  const int rc = plan(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len, partition_tokens, &s);
  if (rc) return rc;
  if (batch == 0) return KVD_OK;
  if (!out || !seq_lens) return KVD_ERR_NULL;
  if (!workspace || workspace_bytes < s.ws.total) return KVD_ERR_WORKSPACE;
  const MergeLaunch m = merge_launch(out, seq_lens, batch, num_q_heads, head_dim, max_seq_len,
                                     workspace, dtype, s);
  return hip_status(launch_merge(m, static_cast<hipStream_t>(stream)));
}

int decode_attn_paged(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_table, const int32_t* seq_lens,
                      int batch, int num_q_heads, int num_kv_heads, int head_dim,
                      int block_size, int max_blocks_per_seq, int num_blocks,
                      int max_seq_len, float scale, int partition_tokens,
                      void* workspace, size_t workspace_bytes, kvd_dtype_t dtype, void* stream) {
  Sizes s;
  int rc = check_paged(q, k_cache, v_cache, block_table, seq_lens, batch, num_q_heads,
                       num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                       max_seq_len, partition_tokens, workspace, workspace_bytes, dtype, &s);
  if (rc) return rc;
  if (batch == 0) return KVD_OK;
  if (!out) return KVD_ERR_NULL;
  rc = preconditions(seq_lens, block_table, nullptr, batch, max_blocks_per_seq, num_blocks,
                     max_seq_len, false,
                     {{q, bytes_of(batch, num_q_heads, head_dim, dtype), dtype}}, stream);
  if (rc) return rc;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const PagedLaunch a = paged_launch(q, k_cache, v_cache, block_table, seq_lens, batch,
                                     num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                                     num_blocks, max_seq_len, scale, workspace, dtype, s);
  rc = hip_status(launch_paged_partials(a, st));
  if (rc) return rc;
  const MergeLaunch m = merge_launch(out, seq_lens, batch, num_q_heads, head_dim, max_seq_len,
                                     workspace, dtype, s);
  return hip_status(launch_merge(m, st));
}

int decode_attn_paged_window_partials(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_table, const int32_t* seq_lens,
                                      int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                      int block_size, int max_blocks_per_seq, int num_blocks,
                                      int max_seq_len, float scale, int window,
                                      int partition_tokens, void* workspace,
                                      size_t workspace_bytes, kvd_dtype_t dtype, void* stream) {
  Sizes s;
  const int rc = check_paged(q, k_cache, v_cache, block_table, seq_lens, batch, num_q_heads,
                             num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                             max_seq_len, partition_tokens, workspace, workspace_bytes, dtype, &s);
  if (rc) return rc;
  if (window < 1) return KVD_ERR_SHAPE;
  if (batch == 0) return KVD_OK;
  const int vc = preconditions(seq_lens, block_table, nullptr, batch, max_blocks_per_seq,
                               num_blocks, max_seq_len, false,
                               {{q, bytes_of(batch, num_q_heads, head_dim, dtype), dtype}}, stream);
  if (vc) return vc;
  PagedLaunch a = paged_launch(q, k_cache, v_cache, block_table, seq_lens, batch, num_q_heads,
                               num_kv_heads, head_dim, max_blocks_per_seq, num_blocks,
                               max_seq_len, scale, workspace, dtype, s);
  a.window = window;
  return hip_status(launch_paged_partials(a, static_cast<hipStream_t>(stream)));
}

int decode_attn_paged_window(void* out, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_table, const int32_t* seq_lens, int batch,
                             int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                             int max_blocks_per_seq, int num_blocks, int max_seq_len,
                             float scale, int window, int partition_tokens, void* workspace,
                             size_t workspace_bytes, kvd_dtype_t dtype, void* stream) {
  Sizes s;
  int rc = check_paged(q, k_cache, v_cache, block_table, seq_lens, batch, num_q_heads,
                       num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                       max_seq_len, partition_tokens, workspace, workspace_bytes, dtype, &s);
  if (rc) return rc;
  if (window < 1) return KVD_ERR_SHAPE;
  if (batch == 0) return KVD_OK;
  if (!out) return KVD_ERR_NULL;
  rc = decode_attn_paged_window_partials(q, k_cache, v_cache, block_table, seq_lens, batch,
                                         num_q_heads, num_kv_heads, head_dim, block_size,
                                         max_blocks_per_seq, num_blocks, max_seq_len, scale,
                                         window, partition_tokens, workspace, workspace_bytes,
                                         dtype, stream);
  if (rc) return rc;
  const MergeLaunch m = merge_launch(out, seq_lens, batch, num_q_heads, head_dim, max_seq_len,
                                     workspace, dtype, s);
  return hip_status(launch_merge(m, static_cast<hipStream_t>(stream)));
}

int decode_attn_paged_append_partials(const void* q, void* k_cache, void* v_cache,
                                      const void* k_new, const void* v_new,
                                      const int32_t* block_table, const int32_t* seq_lens,
                                      int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                      int block_size, int max_blocks_per_seq, int num_blocks,
                                      int max_seq_len, float scale, int partition_tokens,
                                      void* workspace, size_t workspace_bytes, kvd_dtype_t dtype,
                                      void* stream) {
  Sizes s;
  const int rc = check_paged(q, k_cache, v_cache, block_table, seq_lens, batch, num_q_heads,
                             num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                             max_seq_len, partition_tokens, workspace, workspace_bytes, dtype, &s);
  if (rc) return rc;
  if (batch == 0) return KVD_OK;
  if (!k_new || !v_new) return KVD_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new)) return KVD_ERR_SHAPE;
  const size_t nb = bytes_of(batch, num_kv_heads, head_dim, dtype);
  const int vc = preconditions(seq_lens, block_table, nullptr, batch, max_blocks_per_seq,
                               num_blocks, max_seq_len, true,
                               {{q, bytes_of(batch, num_q_heads, head_dim, dtype), dtype},
                                {k_new, nb, dtype},
                                {v_new, nb, dtype}},
                               stream);
  if (vc) return vc;
  PagedLaunch a = paged_launch(q, k_cache, v_cache, block_table, seq_lens, batch, num_q_heads,
                               num_kv_heads, head_dim, max_blocks_per_seq, num_blocks,
                               max_seq_len, scale, workspace, dtype, s);
  a.k_new = k_new;
  a.v_new = v_new;
  return hip_status(launch_paged_partials(a, static_cast<hipStream_t>(stream)));
}

int decode_attn_paged_append(void* out, const void* q, void* k_cache, void* v_cache,
                             const void* k_new, const void* v_new, const int32_t* block_table,
                             const int32_t* seq_lens, int batch, int num_q_heads,
                             int num_kv_heads, int head_dim, int block_size,
                             int max_blocks_per_seq, int num_blocks, int max_seq_len,
                             float scale, int partition_tokens, void* workspace,
                             size_t workspace_bytes, kvd_dtype_t dtype, void* stream) {
  if (batch != 0 && !out) {
    // Let the shared checks report other errors first.
    Sizes s;
    const int rc = check_paged(q, k_cache, v_cache, block_table, seq_lens, batch, num_q_heads,
                               num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                               num_blocks, max_seq_len, partition_tokens, workspace,
                               workspace_bytes, dtype, &s);
    return rc ? rc : KVD_ERR_NULL;
  }
  int rc = decode_attn_paged_append_partials(q, k_cache, v_cache, k_new, v_new, block_table,
                                             seq_lens, batch, num_q_heads, num_kv_heads,
                                             head_dim, block_size, max_blocks_per_seq, num_blocks,
                                             max_seq_len, scale, partition_tokens, workspace,
                                             workspace_bytes, dtype, stream);
  if (rc || batch == 0) return rc;
  return decode_attn_merge(out, seq_lens, batch, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                           partition_tokens, workspace, workspace_bytes, dtype, stream);
}

int decode_attn_paged_append_noalloc(void* out, const void* q, void* k_cache, void* v_cache,
                                     const void* k_new, const void* v_new,
                                     const int32_t* block_table, const int32_t* seq_lens,
                                     int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                     int block_size, int max_blocks_per_seq, int num_blocks,
                                     int max_seq_len, float scale, int partition_tokens,
                                     kvd_dtype_t dtype, void* stream) {
  // The scratch array serves as the workspace; everything else is the
  // checked path of decode_attn_paged_append.  No allocation happens here:
  // the array was placed in device memory when the library was loaded on
  // this device.
  if (batch == 0)
    return decode_attn_paged_append(out, q, k_cache, v_cache, k_new, v_new, block_table,
                                    seq_lens, batch, num_q_heads, num_kv_heads, head_dim,
                                    block_size, max_blocks_per_seq, num_blocks, max_seq_len,
                                    scale, partition_tokens, nullptr, 0, dtype, stream);
  const size_t need = decode_attn_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim,
                                                  max_seq_len, partition_tokens);
  if (need == 0) {
    // Sizes the planner rejects: let the shared checks name the error.
    return decode_attn_paged_append(out, q, k_cache, v_cache, k_new, v_new, block_table,
                                    seq_lens, batch, num_q_heads, num_kv_heads, head_dim,
                                    block_size, max_blocks_per_seq, num_blocks, max_seq_len,
                                    scale, partition_tokens, nullptr, 0, dtype, stream);
  }
  if (need > kNoAllocScratchBytes) return KVD_ERR_WORKSPACE;
  hipError_t e = hipSuccess;
  void* ws = noalloc_scratch(&e);
  if (!ws) return KVD_ERR_HIP;
  return decode_attn_paged_append(out, q, k_cache, v_cache, k_new, v_new, block_table, seq_lens,
                                  batch, num_q_heads, num_kv_heads, head_dim, block_size,
                                  max_blocks_per_seq, num_blocks, max_seq_len, scale,
                                  partition_tokens, ws, kNoAllocScratchBytes, dtype, stream);
}

size_t decode_attn_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

size_t kvd_stream_read_sink_bytes(void) {
  return static_cast<size_t>(stream_read_groups()) * 256 * sizeof(uint32_t);
}

int kvd_stream_read(const void* src, size_t bytes, void* sink, size_t sink_bytes, void* stream) {
  if (bytes == 0) return KVD_OK;
  if (!src || !sink) return KVD_ERR_NULL;
  if (bytes % 16 != 0 || !aligned16(src)) return KVD_ERR_SHAPE;
  if (sink_bytes < kvd_stream_read_sink_bytes()) return KVD_ERR_WORKSPACE;
  return hip_status(launch_stream_read(src, bytes, static_cast<uint32_t*>(sink),
                                       static_cast<hipStream_t>(stream)));
}

size_t kvd_lds_read_sink_bytes(int groups) {
  return groups < 1 ? 0 : static_cast<size_t>(groups) * lds_read_threads() * sizeof(uint32_t);
}

long long kvd_lds_read_bytes(int mode, int groups, int iters) {
  if ((mode != 0 && mode != 1) || groups < 1 || iters < 0) return 0;
  return static_cast<long long>(groups) * lds_read_threads() * iters *
         lds_read_bytes_per_lane_iter(mode);
}

int kvd_lds_read(int mode, int groups, int iters, void* cycles, void* sink, size_t sink_bytes,
                 void* stream) {
  if (mode != 0 && mode != 1) return KVD_ERR_UNSUPPORTED;
  if (groups < 1 || groups > 65535 || iters < 1 || iters > (1 << 24)) return KVD_ERR_SHAPE;
  if (!cycles || !sink) return KVD_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(cycles) & 7u) != 0) return KVD_ERR_SHAPE;
  if (sink_bytes < kvd_lds_read_sink_bytes(groups)) return KVD_ERR_WORKSPACE;
  return hip_status(launch_lds_read(mode, groups, iters, static_cast<unsigned long long*>(cycles),
                                    static_cast<uint32_t*>(sink), static_cast<hipStream_t>(stream)));
}

static int append_bytes(void* k_cache, void* v_cache, float* v_scale, const void* k_new,
                        const void* v_new, const float* k_scale, const int32_t* block_table,
                        const int32_t* seq_lens, int batch, int num_kv_heads, int head_dim,
                        int block_size, int max_blocks_per_seq, int num_blocks, int dtype,
                        bool fp8, void* stream) {
  if (!dtype_ok(dtype)) return KVD_ERR_UNSUPPORTED;
  if (batch < 0 || num_kv_heads < 1) return KVD_ERR_SHAPE;
  if (!(head_dim == 32 || head_dim == 64 || head_dim == 128)) return KVD_ERR_UNSUPPORTED;
  if (block_size != kBlockSize) return KVD_ERR_UNSUPPORTED;
  if (max_blocks_per_seq < 1 || max_blocks_per_seq > kMaxTableBlocks || num_blocks < 1)
    return KVD_ERR_SHAPE;
  if (batch == 0) return KVD_OK;
  if (!k_cache || !v_cache || !v_scale || !k_new || !v_new || !k_scale || !block_table ||
      !seq_lens)
    return KVD_ERR_NULL;
  AppendInt8Launch a;
  a.k_cache = static_cast<int8_t*>(k_cache);
  a.v_cache = static_cast<int8_t*>(v_cache);
  a.v_scale = v_scale;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_scale = k_scale;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.batch = batch;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.bf16 = dtype == KVD_BF16;
  a.fp8 = fp8;
  const size_t nb = bytes_of(batch, num_kv_heads, head_dim, dtype);
  const int rc = preconditions(seq_lens, block_table, nullptr, batch, max_blocks_per_seq,
                               num_blocks, 0, true, {{k_new, nb, dtype}, {v_new, nb, dtype}},
                               stream);
  if (rc) return rc;
  return hip_status(launch_append_int8(a, static_cast<hipStream_t>(stream)));
}

int kv_append_paged_int8(int8_t* k_cache, int8_t* v_cache, float* v_scale, const void* k_new,
                         const void* v_new, const float* k_scale, const int32_t* block_table,
                         const int32_t* seq_lens, int batch, int num_kv_heads, int head_dim,
                         int block_size, int max_blocks_per_seq, int num_blocks,
                         kvd_dtype_t dtype, void* stream) {
  return append_bytes(k_cache, v_cache, v_scale, k_new, v_new, k_scale, block_table, seq_lens,
                      batch, num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                      dtype, false, stream);
}

int kv_append_paged_fp8(uint8_t* k_cache, uint8_t* v_cache, float* v_scale, const void* k_new,
                        const void* v_new, const float* k_scale, const int32_t* block_table,
                        const int32_t* seq_lens, int batch, int num_kv_heads, int head_dim,
                        int block_size, int max_blocks_per_seq, int num_blocks,
                        kvd_dtype_t dtype, void* stream) {
  return append_bytes(k_cache, v_cache, v_scale, k_new, v_new, k_scale, block_table, seq_lens,
                      batch, num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                      dtype, true, stream);
}

// The INT8 decode takes bf16 queries (and writes a bf16 output); its scales
// are fp32, the per-channel K scales read 16 bytes at a time.
static int check_paged_int8(const void* q, const void* k_cache, const void* v_cache,
                            const float* k_scale, const float* v_scale,
                            const int32_t* block_table, const int32_t* seq_lens, int batch,
                            int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                            int max_blocks_per_seq, int num_blocks, int max_seq_len,
                            int partition_tokens, const void* workspace, size_t workspace_bytes,
                            int dtype, Sizes* s) {
  if (dtype != KVD_BF16) return KVD_ERR_UNSUPPORTED;
  const int rc = check_paged(q, k_cache, v_cache, block_table, seq_lens, batch, num_q_heads,
                             num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                             max_seq_len, partition_tokens, workspace, workspace_bytes, dtype, s);
  if (rc || batch == 0) return rc;
  if (!k_scale || !v_scale) return KVD_ERR_NULL;
  if (!aligned16(k_scale) || (reinterpret_cast<uintptr_t>(v_scale) & 3u) != 0) return KVD_ERR_SHAPE;
  return KVD_OK;
}

static int bytes_partials(const void* q, const void* k_cache, const void* v_cache,
                          const float* k_scale, const float* v_scale,
                          const int32_t* block_table, const int32_t* seq_lens, int batch,
                          int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                          int max_blocks_per_seq, int num_blocks, int max_seq_len, float scale,
                          int partition_tokens, void* workspace, size_t workspace_bytes,
                          int dtype, bool fp8, void* stream) {
  Sizes s;
  const int rc = check_paged_int8(q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens,
                                  batch, num_q_heads, num_kv_heads, head_dim, block_size,
                                  max_blocks_per_seq, num_blocks, max_seq_len, partition_tokens,
                                  workspace, workspace_bytes, dtype, &s);
  if (rc || batch == 0) return rc;
  const int vc = preconditions(seq_lens, block_table, nullptr, batch, max_blocks_per_seq,
                               num_blocks, max_seq_len, false,
                               {{q, bytes_of(batch, num_q_heads, head_dim, dtype), dtype}}, stream);
  if (vc) return vc;
  PagedLaunch a = paged_launch(q, k_cache, v_cache, block_table, seq_lens, batch, num_q_heads,
                               num_kv_heads, head_dim, max_blocks_per_seq, num_blocks,
                               max_seq_len, scale, workspace, dtype, s);
  a.int8 = true;
  a.fp8 = fp8;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  return hip_status(launch_paged_partials(a, static_cast<hipStream_t>(stream)));
}

int decode_attn_paged_int8_partials(const void* q, const int8_t* k_cache, const int8_t* v_cache,
                                    const float* k_scale, const float* v_scale,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                    int block_size, int max_blocks_per_seq, int num_blocks,
                                    int max_seq_len, float scale, int partition_tokens,
                                    void* workspace, size_t workspace_bytes, kvd_dtype_t dtype,
                                    void* stream) {
  return bytes_partials(q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens, batch,
                        num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                        num_blocks, max_seq_len, scale, partition_tokens, workspace,
                        workspace_bytes, dtype, false, stream);
}

int decode_attn_paged_fp8_partials(const void* q, const uint8_t* k_cache, const uint8_t* v_cache,
                                   const float* k_scale, const float* v_scale,
                                   const int32_t* block_table, const int32_t* seq_lens,
                                   int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                   int block_size, int max_blocks_per_seq, int num_blocks,
                                   int max_seq_len, float scale, int partition_tokens,
                                   void* workspace, size_t workspace_bytes, kvd_dtype_t dtype,
                                   void* stream) {
  return bytes_partials(q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens, batch,
                        num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                        num_blocks, max_seq_len, scale, partition_tokens, workspace,
                        workspace_bytes, dtype, true, stream);
}

static int bytes_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                        const float* k_scale, const float* v_scale,
                        const int32_t* block_table, const int32_t* seq_lens, int batch,
                        int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                        int max_blocks_per_seq, int num_blocks, int max_seq_len, float scale,
                        int partition_tokens, void* workspace, size_t workspace_bytes, int dtype,
                        bool fp8, void* stream) {
  Sizes s;
  int rc = check_paged_int8(q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens, batch,
                            num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                            num_blocks, max_seq_len, partition_tokens, workspace,
                            workspace_bytes, dtype, &s);
  if (rc || batch == 0) return rc;
  if (!out) return KVD_ERR_NULL;
  rc = bytes_partials(q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens, batch,
                      num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                      num_blocks, max_seq_len, scale, partition_tokens, workspace,
                      workspace_bytes, dtype, fp8, stream);
  if (rc) return rc;
  const MergeLaunch m = merge_launch(out, seq_lens, batch, num_q_heads, head_dim, max_seq_len,
                                     workspace, dtype, s);
  return hip_status(launch_merge(m, static_cast<hipStream_t>(stream)));
}

int decode_attn_paged_int8(void* out, const void* q, const int8_t* k_cache, const int8_t* v_cache,
                           const float* k_scale, const float* v_scale,
                           const int32_t* block_table, const int32_t* seq_lens, int batch,
                           int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                           int max_blocks_per_seq, int num_blocks, int max_seq_len, float scale,
                           int partition_tokens, void* workspace, size_t workspace_bytes,
                           kvd_dtype_t dtype, void* stream) {
  return bytes_decode(out, q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens, batch,
                      num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                      num_blocks, max_seq_len, scale, partition_tokens, workspace,
                      workspace_bytes, dtype, false, stream);
}

int decode_attn_paged_fp8(void* out, const void* q, const uint8_t* k_cache,
                          const uint8_t* v_cache, const float* k_scale, const float* v_scale,
                          const int32_t* block_table, const int32_t* seq_lens, int batch,
                          int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                          int max_blocks_per_seq, int num_blocks, int max_seq_len, float scale,
                          int partition_tokens, void* workspace, size_t workspace_bytes,
                          kvd_dtype_t dtype, void* stream) {
  return bytes_decode(out, q, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens, batch,
                      num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                      num_blocks, max_seq_len, scale, partition_tokens, workspace,
                      workspace_bytes, dtype, true, stream);
}

int kv_copy_blocks(void* cache, const int32_t* pairs, int num_pairs, size_t block_bytes,
                   int num_blocks, void* stream) {
  if (num_pairs < 0 || num_blocks < 1 || block_bytes == 0 || block_bytes % 4 != 0)
    return KVD_ERR_SHAPE;
  if (num_pairs == 0) return KVD_OK;
  if (!cache || !pairs) return KVD_ERR_NULL;
  CopyBlocksLaunch a;
  a.cache = cache;
  a.pairs = pairs;
  a.num_pairs = num_pairs;
  a.num_blocks = num_blocks;
  a.block_bytes = block_bytes;
  a.vec16 = aligned16(cache) && block_bytes % 16 == 0;
  return hip_status(launch_copy_blocks(a, static_cast<hipStream_t>(stream)));
}

int kv_append_paged_multi(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                          const int32_t* cu_rows, const int32_t* block_table,
                          const int32_t* seq_lens, int batch, int max_rows, int num_kv_heads,
                          int head_dim, int block_size, int max_blocks_per_seq, int num_blocks,
                          kvd_dtype_t dtype, void* stream) {
  if (!dtype_ok(dtype)) return KVD_ERR_UNSUPPORTED;
  if (batch < 0 || max_rows < 0 || num_kv_heads < 1 || head_dim < 1 || head_dim > 1024)
    return KVD_ERR_SHAPE;
  if (block_size != kBlockSize) return KVD_ERR_UNSUPPORTED;
  if (max_blocks_per_seq < 1 || max_blocks_per_seq > kMaxTableBlocks || num_blocks < 1)
    return KVD_ERR_SHAPE;
  const long long row_bytes = static_cast<long long>(num_kv_heads) * head_dim * elem_bytes(dtype);
  if (row_bytes % 4 != 0 || row_bytes / 4 > INT_MAX) return KVD_ERR_SHAPE;
  if (batch == 0 || max_rows == 0) return KVD_OK;
  if (batch > 65535 || max_rows > INT_MAX / 2) return KVD_ERR_SHAPE;
  if (!k_cache || !v_cache || !k_new || !v_new || !cu_rows || !block_table || !seq_lens)
    return KVD_ERR_NULL;
  AppendMultiLaunch a;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_new = k_new;
  a.v_new = v_new;
  a.cu_rows = cu_rows;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.batch = batch;
  a.max_rows = max_rows;
  a.row_words = static_cast<int>(row_bytes / 4);
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.vec16 = aligned16(k_cache) && aligned16(v_cache) && aligned16(k_new) && aligned16(v_new);
  const int rc = preconditions(seq_lens, block_table, cu_rows, batch, max_blocks_per_seq,
                               num_blocks, 0, false, {}, stream);
  if (rc) return rc;
  return hip_status(launch_append_multi(a, static_cast<hipStream_t>(stream)));
}

int prefill_attn_paged(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* cu_rows, const int32_t* block_table,
                       const int32_t* seq_lens, int batch, int max_rows, int num_q_heads,
                       int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                       int num_blocks, int max_seq_len, float scale, kvd_dtype_t dtype,
                       void* stream) {
  if (!dtype_ok(dtype)) return KVD_ERR_UNSUPPORTED;
  int rc = check_heads(batch, num_q_heads, num_kv_heads);
  if (rc) return rc;
  if (!prefill_supported(head_dim, dtype == KVD_BF16)) return KVD_ERR_UNSUPPORTED;
  rc = check_table(block_size, max_blocks_per_seq, num_blocks, max_seq_len);
  if (rc) return rc;
  if (max_rows < 0 || max_rows > max_seq_len) return KVD_ERR_SHAPE;
  if (batch > 65535 || num_kv_heads > 65535) return KVD_ERR_SHAPE;
  const long long r = num_q_heads / num_kv_heads;
  if ((static_cast<long long>(max_rows) * r + 63) / 64 > INT_MAX) return KVD_ERR_SHAPE;
  if (batch == 0 || max_rows == 0) return KVD_OK;
  if (!out || !q || !k_cache || !v_cache || !cu_rows || !block_table || !seq_lens)
    return KVD_ERR_NULL;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return KVD_ERR_SHAPE;
  rc = preconditions(seq_lens, block_table, nullptr, batch, max_blocks_per_seq, num_blocks,
                     max_seq_len, false, {}, stream);
  if (rc) return rc;
  PrefillLaunch a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.cu_rows = cu_rows;
  a.out = out;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.max_seq_len = max_seq_len;
  a.max_rows = max_rows;
  a.scale = scale;
  return hip_status(launch_prefill(a, static_cast<hipStream_t>(stream)));
}

static int mla_setup(const void* q, const void* c_cache, const int32_t* block_table,
                     const int32_t* seq_lens, int batch, int num_q_heads, int d_c, int d_rope,
                     int block_size, int max_blocks_per_seq, int num_blocks, int max_seq_len,
                     float scale, int partition_tokens, void* workspace, size_t workspace_bytes,
                     Sizes* s, MlaLaunch* a) {
  if (batch < 0 || num_q_heads < 1) return KVD_ERR_SHAPE;
  if (!mla_supported(num_q_heads, d_c, d_rope)) return KVD_ERR_UNSUPPORTED;
  int rc = check_table(block_size, max_blocks_per_seq, num_blocks, max_seq_len);
  if (rc) return rc;
  // Tiles are 32 tokens: an explicit partition must be a multiple of 32.
  if (partition_tokens > 0 && partition_tokens % 32 != 0) return KVD_ERR_SHAPE;
  rc = plan(batch, num_q_heads, 1, d_c, max_seq_len, partition_tokens, s);
  if (rc) return rc;
  if (batch == 0) return KVD_OK;
  if (!q || !c_cache || !block_table || !seq_lens) return KVD_ERR_NULL;
  if (!workspace || workspace_bytes < s->ws.total) return KVD_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(c_cache) || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return KVD_ERR_SHAPE;
  a->q = q;
  a->c_cache = c_cache;
  a->block_table = block_table;
  a->seq_lens = seq_lens;
  a->ws_o = static_cast<float*>(workspace);
  a->ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + s->ws.ml_offset);
  a->batch = batch;
  a->num_heads = num_q_heads;
  a->max_blocks_per_seq = max_blocks_per_seq;
  a->num_blocks = num_blocks;
  a->max_seq_len = max_seq_len;
  a->partition_tokens = s->pt;
  a->num_partitions = s->parts;
  a->scale = scale;
  a->c_new = nullptr;
  return KVD_OK;
}

int decode_attn_mla_partials(const void* q, const void* c_cache,
                             const int32_t* block_table, const int32_t* seq_lens,
                             int batch, int num_q_heads, int d_c, int d_rope, int block_size,
                             int max_blocks_per_seq, int num_blocks, int max_seq_len,
                             float scale, int partition_tokens, void* workspace,
                             size_t workspace_bytes, void* stream) {
  Sizes s;
  MlaLaunch a;
  const int rc = mla_setup(q, c_cache, block_table, seq_lens, batch, num_q_heads, d_c, d_rope,
                           block_size, max_blocks_per_seq, num_blocks, max_seq_len, scale,
                           partition_tokens, workspace, workspace_bytes, &s, &a);
  if (rc || batch == 0) return rc;
  const int vc = preconditions(seq_lens, block_table, nullptr, batch, max_blocks_per_seq,
                               num_blocks, max_seq_len, false,
                               {{q, bytes_of(batch, num_q_heads, d_c + d_rope, KVD_BF16), KVD_BF16}},
                               stream);
  if (vc) return vc;
  return hip_status(launch_mla_partials(a, static_cast<hipStream_t>(stream)));
}

int decode_attn_mla(void* out, const void* q, const void* c_cache,
                    const int32_t* block_table, const int32_t* seq_lens,
                    int batch, int num_q_heads, int d_c, int d_rope, int block_size,
                    int max_blocks_per_seq, int num_blocks, int max_seq_len, float scale,
                    int partition_tokens, void* workspace, size_t workspace_bytes,
                    void* stream) {
  Sizes s;
  MlaLaunch a;
  int rc = mla_setup(q, c_cache, block_table, seq_lens, batch, num_q_heads, d_c, d_rope,
                     block_size, max_blocks_per_seq, num_blocks, max_seq_len, scale,
                     partition_tokens, workspace, workspace_bytes, &s, &a);
  if (rc || batch == 0) return rc;
  if (!out) return KVD_ERR_NULL;
  rc = preconditions(seq_lens, block_table, nullptr, batch, max_blocks_per_seq, num_blocks,
                     max_seq_len, false,
                     {{q, bytes_of(batch, num_q_heads, d_c + d_rope, KVD_BF16), KVD_BF16}}, stream);
  if (rc) return rc;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  rc = hip_status(launch_mla_partials(a, st));
  if (rc) return rc;
  const MergeLaunch m = merge_launch(out, seq_lens, batch, num_q_heads, d_c, max_seq_len,
                                     workspace, KVD_BF16, s);
  return hip_status(launch_merge(m, st));
}

// MLA with the append fused in: the checks of decode_attn_mla plus the new
// rows; launches the partials (and the merge when `out` is given).
static int mla_append_impl(void* out, const void* q, void* c_cache, const void* c_new,
                           const int32_t* block_table, const int32_t* seq_lens, int batch,
                           int num_q_heads, int d_c, int d_rope, int block_size,
                           int max_blocks_per_seq, int num_blocks, int max_seq_len, float scale,
                           int partition_tokens, void* workspace, size_t workspace_bytes,
                           void* stream, bool merge) {
  Sizes s;
  MlaLaunch a;
  int rc = mla_setup(q, c_cache, block_table, seq_lens, batch, num_q_heads, d_c, d_rope,
                     block_size, max_blocks_per_seq, num_blocks, max_seq_len, scale,
                     partition_tokens, workspace, workspace_bytes, &s, &a);
  if (rc || batch == 0) return rc;
  if (!c_new || (merge && !out)) return KVD_ERR_NULL;
  if (!aligned16(c_new)) return KVD_ERR_SHAPE;
  rc = preconditions(seq_lens, block_table, nullptr, batch, max_blocks_per_seq, num_blocks,
                     max_seq_len, true,
                     {{q, bytes_of(batch, num_q_heads, d_c + d_rope, KVD_BF16), KVD_BF16},
                      {c_new, bytes_of(batch, 1, d_c + d_rope, KVD_BF16), KVD_BF16}},
                     stream);
  if (rc) return rc;
  a.c_new = c_new;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  rc = hip_status(launch_mla_partials(a, st));
  if (rc || !merge) return rc;
  const MergeLaunch m = merge_launch(out, seq_lens, batch, num_q_heads, d_c, max_seq_len,
                                     workspace, KVD_BF16, s);
  return hip_status(launch_merge(m, st));
}

int decode_attn_mla_append_partials(const void* q, void* c_cache, const void* c_new,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    int batch, int num_q_heads, int d_c, int d_rope,
                                    int block_size, int max_blocks_per_seq, int num_blocks,
                                    int max_seq_len, float scale, int partition_tokens,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  return mla_append_impl(nullptr, q, c_cache, c_new, block_table, seq_lens, batch, num_q_heads,
                         d_c, d_rope, block_size, max_blocks_per_seq, num_blocks, max_seq_len,
                         scale, partition_tokens, workspace, workspace_bytes, stream, false);
}

int decode_attn_mla_append(void* out, const void* q, void* c_cache, const void* c_new,
                           const int32_t* block_table, const int32_t* seq_lens, int batch,
                           int num_q_heads, int d_c, int d_rope, int block_size,
                           int max_blocks_per_seq, int num_blocks, int max_seq_len, float scale,
                           int partition_tokens, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return mla_append_impl(out, q, c_cache, c_new, block_table, seq_lens, batch, num_q_heads, d_c,
                         d_rope, block_size, max_blocks_per_seq, num_blocks, max_seq_len, scale,
                         partition_tokens, workspace, workspace_bytes, stream, true);
}


}  // extern "C"
