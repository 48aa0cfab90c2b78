// Host-side interfaces between the C ABI layer (api.cpp) and the kernel
// launchers (*.hip).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace kvd {

// Workspace of the split decode: per (b, h, partition) an fp32 output row of
// head_dim values, then per (b, h, partition) the pair (max, sum).  The max is
// kept in log2 units (scores are pre-multiplied by log2 e).
// With the balanced split P is the bound on the pieces of one (b, h) and a
// third array holds, per (b, h), the number of pieces written.
struct WorkspaceLayout {
  size_t o_bytes;        // [B, H_q, P, D] fp32
  size_t ml_offset;      // start of [B, H_q, P] float2, 256-B aligned
  size_t counts_offset;  // start of [B, H_q] int32 piece counts (balanced split only)
  size_t total;
};

WorkspaceLayout workspace_layout(int batch, int num_q_heads, int num_partitions, int head_dim,
                                 bool balanced);

// Smallest piece of the balanced split, in 16-token blocks.
constexpr int kBalancedMinPieceBlocks = 16;

struct PagedLaunch {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  float* ws_o;
  float* ws_ml;
  int batch, num_q_heads, num_kv_heads, head_dim;
  int max_blocks_per_seq, num_blocks, max_seq_len;
  int partition_tokens, num_partitions;
  float scale;
  bool bf16;
  int* counts;  // balanced split: piece counts per (b, h); NULL for fixed partitions
  // Fused append: this step's K/V rows [B, H_kv, D] (both NULL otherwise);
  // k_cache / v_cache are then written (the new rows' slots only).
  const void* k_new;
  const void* v_new;
  // INT8 cache: k_cache / v_cache hold codes, k_scale [H_kv, D] the
  // per-channel K scales, v_scale [NB, 16, H_kv] the per-token V scales;
  // q and the output are bf16.
  bool int8;
  bool fp8;  // with int8: the codes are FP8 E4M3, not integers
  const float* k_scale;
  const float* v_scale;
  // Sliding window: each row sees its last `window` positions; 0 = all.
  int window;
};

struct MergeLaunch {
  void* out;
  const int32_t* seq_lens;
  const float* ws_o;
  const float* ws_ml;
  int batch, num_q_heads, head_dim;
  int max_blocks_per_seq_tokens;  // clamp bound for seq_lens (max_seq_len)
  int partition_tokens, num_partitions;
  bool bf16;
  const int* counts;  // balanced split: piece counts per (b, h); NULL for fixed partitions
};

struct AppendLaunch {
  void* k_cache;
  void* v_cache;
  const void* k_new;
  const void* v_new;
  const int32_t* block_table;
  const int32_t* seq_lens;
  int batch, row_words;  // row_words = num_kv_heads * head_dim * elem / 4
  int max_blocks_per_seq, num_blocks;
  bool vec16;  // all four row buffers 16-byte aligned
};

struct AppendInt8Launch {
  int8_t* k_cache;        // [NB, 16, H_kv, D] codes
  int8_t* v_cache;        // [NB, 16, H_kv, D] codes
  float* v_scale;         // [NB, 16, H_kv]
  const void* k_new;      // [B, H_kv, D] bf16 or fp32
  const void* v_new;
  const float* k_scale;   // [H_kv, D]
  const int32_t* block_table;
  const int32_t* seq_lens;
  int batch, num_kv_heads, head_dim, max_blocks_per_seq, num_blocks;
  bool bf16;
  bool fp8;  // E4M3 codes (V scale max |v| / 448) instead of INT8 codes
};

struct CopyBlocksLaunch {
  void* cache;
  const int32_t* pairs;  // device [num_pairs][2]
  int num_pairs, num_blocks;
  size_t block_bytes;
  bool vec16;  // cache 16-byte aligned and block_bytes a multiple of 16
};

struct PrefillLaunch {
  const void* q;            // [N, H_q, D] bf16, rows of sequence b are cu_rows[b] ..
  const void* k_cache;      // [NB, 16, H_kv, D] bf16
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;  // positions including the new rows
  const int32_t* cu_rows;   // [B + 1]
  void* out;                // [N, H_q, D] bf16
  int batch, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, num_blocks, max_seq_len;
  int max_rows;             // bound on rows per sequence (sizes the grid)
  float scale;
};

struct AppendMultiLaunch {
  void* k_cache;
  void* v_cache;
  const void* k_new;        // [N, H_kv, D]
  const void* v_new;
  const int32_t* cu_rows;
  const int32_t* block_table;
  const int32_t* seq_lens;
  int batch, max_rows, row_words, max_blocks_per_seq, num_blocks;
  bool vec16;
};

struct MlaLaunch {
  const void* q;            // [B, H, d_c + d_rope] bf16
  const void* c_cache;      // [NB, 16, d_c + d_rope] bf16
  const int32_t* block_table;
  const int32_t* seq_lens;
  float* ws_o;
  float* ws_ml;
  int batch, num_heads, max_blocks_per_seq, num_blocks, max_seq_len;
  int partition_tokens, num_partitions;
  float scale;
  // Fused append: this step's rows [B, d_c + d_rope] (NULL otherwise);
  // c_cache is then written (the new rows' slots only).
  const void* c_new;
};

// Allocation-free entry point: size of the per-device scratch array that
// stands in for the caller's workspace (64 MiB), and its device address on
// the current device (looked up once per device; NULL and *err set on a HIP
// error).
constexpr size_t kNoAllocScratchBytes = static_cast<size_t>(64) << 20;
void* noalloc_scratch(hipError_t* err);

// Streaming-read probe: workgroups launched (the sink holds one word per
// thread of them), and the launch over `bytes` (a multiple of 16).
int stream_read_groups();
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

// Each returns hipSuccess or the launch error.
hipError_t launch_append(const AppendLaunch& a, hipStream_t stream);
hipError_t launch_append_int8(const AppendInt8Launch& a, hipStream_t stream);
hipError_t launch_copy_blocks(const CopyBlocksLaunch& a, hipStream_t stream);
hipError_t launch_append_multi(const AppendMultiLaunch& a, hipStream_t stream);
hipError_t launch_prefill(const PrefillLaunch& a, hipStream_t stream);
bool prefill_supported(int head_dim, bool bf16);
hipError_t launch_paged_partials(const PagedLaunch& a, hipStream_t stream);
hipError_t launch_merge(const MergeLaunch& a, hipStream_t stream);
hipError_t launch_mla_partials(const MlaLaunch& a, hipStream_t stream);

// Whether a kernel instance exists for this head_dim / group ratio / dtype.
bool paged_supported(int head_dim, int ratio, bool bf16);
bool mla_supported(int num_heads, int d_c, int d_rope);
// Workgroups per (sequence, partition): one per 64 query heads.
int mla_head_groups(int num_heads);

}  // namespace kvd
