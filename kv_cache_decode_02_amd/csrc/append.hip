// kv_append_paged kernel: copy each sequence's new K/V row into its slot.
//
// Position seq_lens[b] - 1 of sequence b lives in physical block
// block_table[b][pos / 16] at offset pos % 16; the row there is
// num_kv_heads * head_dim values, copied as raw 32-bit words so the write is
// bit-exact for any element type.  This is the preallocated in-place write of
// the "单请求 KV Cache" tutorial (生产系统的做法：预分配 + in-place 写入),
// addressed through the block table of "KV-Cache——为什么AI回复越来越快"
// (08 PagedAttention（vLLM）).
#include "kvd_device.h"
#include "kvd_internal.h"

namespace kvd {
namespace {

template <int VEC>
__global__ __launch_bounds__(256) void append_kernel(AppendLaunch a) {
  const int b = blockIdx.x;
  const bool is_v = blockIdx.y == 1;
  uint32_t* cache = static_cast<uint32_t*>(is_v ? a.v_cache : a.k_cache);
  const uint32_t* src = static_cast<const uint32_t*>(is_v ? a.v_new : a.k_new);
  if (cache == nullptr) return;

  const int len = a.seq_lens[b];
  const long long cap = static_cast<long long>(a.max_blocks_per_seq) * kBlockTokens;
  if (len < 1 || len > cap) return;  // violated precondition: write nothing
  const int pos = len - 1;
  const int blk = a.block_table[static_cast<size_t>(b) * a.max_blocks_per_seq + pos / kBlockTokens];
  if (blk < 0 || blk >= a.num_blocks) return;

  const size_t row = static_cast<size_t>(blk) * kBlockTokens + pos % kBlockTokens;
  uint32_t* dst = cache + row * a.row_words;
  const uint32_t* s = src + static_cast<size_t>(b) * a.row_words;
  for (int w = threadIdx.x * VEC; w < a.row_words; w += blockDim.x * VEC) {
    uint32_t tmp[VEC];
    load_words<VEC>(tmp, s + w);
    store_words<VEC>(dst + w, tmp);
  }
}

}  // namespace

hipError_t launch_append(const AppendLaunch& a, hipStream_t stream) {
  dim3 grid(a.batch, a.v_cache ? 2 : 1);
  if (a.vec16 && a.row_words % 4 == 0) {
    hipLaunchKernelGGL(append_kernel<4>, grid, dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(append_kernel<1>, grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace kvd
