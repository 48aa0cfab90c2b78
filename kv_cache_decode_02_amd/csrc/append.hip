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

// INT8 cache ("KV-Cache——为什么AI回复越来越快", KV-Cache量化: K per channel, V
// per token): code = clip(round_half_even(x / s), -127, 127), every step in
// fp32 with correctly rounded divisions; K takes the caller's per-channel
// scales, V the scale max |v| / 127 of its own row (0 and all codes 0 for a
// zero row), stored beside the codes.  One wave per (sequence, KV head);
// lane l handles dimensions l, l + 64, ...
__device__ __forceinline__ int8_t quantize_code(float x, float s) {
  if (!(s > 0.f)) return 0;
  const float r = rintf(__fdiv_rn(x, s));
  return static_cast<int8_t>(fminf(fmaxf(r, -127.f), 127.f));
}

// FP8 cache: the E4M3 byte (OCP 8-bit float: bias 7, 3 mantissa bits,
// subnormals, largest finite 448) nearest to y, ties to the even code,
// magnitudes past 448 saturating, with y's sign bit.  Subnormal range
// (|y| < 2^-6): the count of 2^-9 steps, rint(|y| * 512) (exact scaling,
// round half to even), whose codes 0 .. 8 run on into the normal ones.
// Normal range: |y|'s fp32 pattern rounded to 3 mantissa bits, half to
// even, then re-biased from 127 to 7 (the carry of a round-up moves into
// the exponent, as the E4M3 pattern needs).
__device__ __forceinline__ uint8_t e4m3_code(float y) {
  const uint32_t bits = __float_as_uint(y);
  const float a = fabsf(y);
  uint32_t mag;
  if (a >= 448.f) {
    mag = 0x7E;
  } else if (a < 0.015625f) {
    mag = static_cast<uint32_t>(rintf(a * 512.f));
  } else {
    const uint32_t u = bits & 0x7FFFFFFFu;
    const uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);
    mag = (r >> 20) - (120u << 3);
  }
  return static_cast<uint8_t>(mag | ((bits >> 24) & 0x80u));
}

template <bool FP8>
__device__ __forceinline__ int8_t quantize_byte(float x, float s) {
  if constexpr (FP8) {
    if (!(s > 0.f)) return 0;
    return static_cast<int8_t>(e4m3_code(__fdiv_rn(x, s)));
  } else {
    return quantize_code(x, s);
  }
}

template <bool BF16, int D, bool FP8>
__global__ __launch_bounds__(256) void append_int8_kernel(AppendInt8Launch a) {
  constexpr int EPL = (D + kWave - 1) / kWave;  // elements per lane
  const int b = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const int len = a.seq_lens[b];
  const long long cap = static_cast<long long>(a.max_blocks_per_seq) * kBlockTokens;
  if (len < 1 || len > cap) return;  // violated precondition: write nothing
  const int pos = len - 1;
  const int blk = a.block_table[static_cast<size_t>(b) * a.max_blocks_per_seq + pos / kBlockTokens];
  if (blk < 0 || blk >= a.num_blocks) return;
  const size_t row = static_cast<size_t>(blk) * kBlockTokens + pos % kBlockTokens;

  for (int g = threadIdx.x >> 6; g < a.num_kv_heads; g += blockDim.x >> 6) {
    const size_t src = (static_cast<size_t>(b) * a.num_kv_heads + g) * D;
    const size_t dst = (row * a.num_kv_heads + g) * D;
    float kx[EPL], vx[EPL];
    float vmax = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int j = lane + i * kWave;
      kx[i] = vx[i] = 0.f;
      if (j < D) {
        if constexpr (BF16) {
          kx[i] = __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(a.k_new)[src + j]) << 16);
          vx[i] = __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(a.v_new)[src + j]) << 16);
        } else {
          kx[i] = static_cast<const float*>(a.k_new)[src + j];
          vx[i] = static_cast<const float*>(a.v_new)[src + j];
        }
        vmax = fmaxf(vmax, fabsf(vx[i]));
      }
    }
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) vmax = fmaxf(vmax, shfl_xor_f(vmax, sh));
    const float vs = __fdiv_rn(vmax, FP8 ? 448.f : 127.f);
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int j = lane + i * kWave;
      if (j < D) {
        a.k_cache[dst + j] = quantize_byte<FP8>(kx[i], a.k_scale[static_cast<size_t>(g) * D + j]);
        a.v_cache[dst + j] = quantize_byte<FP8>(vx[i], vs);
      }
    }
    if (lane == 0) a.v_scale[row * a.num_kv_heads + g] = vs;
  }
}

template <bool BF16, bool FP8>
hipError_t launch_append_int8_typed(const AppendInt8Launch& a, hipStream_t stream) {
  const dim3 grid(a.batch), block(256);
  switch (a.head_dim) {
    case 32: hipLaunchKernelGGL((append_int8_kernel<BF16, 32, FP8>), grid, block, 0, stream, a); break;
    case 64: hipLaunchKernelGGL((append_int8_kernel<BF16, 64, FP8>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((append_int8_kernel<BF16, 128, FP8>), grid, block, 0, stream, a); break;
  }
  return hipGetLastError();
}

// Whole-block copies for copy-on-write: workgroup i copies pair i, as 16-byte
// words when the block size allows, else 4-byte words.
template <int VEC>
__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyBlocksLaunch a) {
  const int32_t src = a.pairs[2 * blockIdx.x], dst = a.pairs[2 * blockIdx.x + 1];
  if (src < 0 || src >= a.num_blocks || dst < 0 || dst >= a.num_blocks) return;
  const size_t words = a.block_bytes / 4;
  const uint32_t* s = static_cast<const uint32_t*>(a.cache) + static_cast<size_t>(src) * words;
  uint32_t* d = static_cast<uint32_t*>(a.cache) + static_cast<size_t>(dst) * words;
  for (size_t w = threadIdx.x * VEC; w < words; w += blockDim.x * VEC) {
    uint32_t tmp[VEC];
    load_words<VEC>(tmp, s + w);
    store_words<VEC>(d + w, tmp);
  }
}

// Many-slot append: workgroup (i, b, tensor) writes new row i of sequence b
// to position seq_lens[b] - n_b + i.
template <int VEC>
__global__ __launch_bounds__(256) void append_multi_kernel(AppendMultiLaunch a) {
  const int i = blockIdx.x, b = blockIdx.y;
  const bool is_v = blockIdx.z == 1;
  const int r0 = a.cu_rows[b];
  const int n = a.cu_rows[b + 1] - r0;
  if (i >= n) return;
  const int len = a.seq_lens[b];
  const long long cap = static_cast<long long>(a.max_blocks_per_seq) * kBlockTokens;
  if (n > len || len > cap) return;  // violated precondition: write nothing
  const int pos = len - n + i;
  const int blk = a.block_table[static_cast<size_t>(b) * a.max_blocks_per_seq + pos / kBlockTokens];
  if (blk < 0 || blk >= a.num_blocks) return;
  uint32_t* cache = static_cast<uint32_t*>(is_v ? a.v_cache : a.k_cache);
  const uint32_t* src = static_cast<const uint32_t*>(is_v ? a.v_new : a.k_new) +
                        static_cast<size_t>(r0 + i) * a.row_words;
  uint32_t* dst = cache + (static_cast<size_t>(blk) * kBlockTokens + pos % kBlockTokens) * a.row_words;
  for (int w = threadIdx.x * VEC; w < a.row_words; w += blockDim.x * VEC) {
    uint32_t tmp[VEC];
    load_words<VEC>(tmp, src + w);
    store_words<VEC>(dst + w, tmp);
  }
}

}  // namespace

hipError_t launch_append_multi(const AppendMultiLaunch& a, hipStream_t stream) {
  const dim3 grid(a.max_rows, a.batch, 2);
  if (a.vec16 && a.row_words % 4 == 0) {
    hipLaunchKernelGGL(append_multi_kernel<4>, grid, dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(append_multi_kernel<1>, grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const CopyBlocksLaunch& a, hipStream_t stream) {
  if (a.vec16) {
    hipLaunchKernelGGL(copy_blocks_kernel<4>, dim3(a.num_pairs), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(copy_blocks_kernel<1>, dim3(a.num_pairs), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_append_int8(const AppendInt8Launch& a, hipStream_t stream) {
  if (a.fp8)
    return a.bf16 ? launch_append_int8_typed<true, true>(a, stream)
                  : launch_append_int8_typed<false, true>(a, stream);
  return a.bf16 ? launch_append_int8_typed<true, false>(a, stream)
                : launch_append_int8_typed<false, false>(a, stream);
}

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
