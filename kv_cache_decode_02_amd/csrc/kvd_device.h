// Device helpers shared by the gfx950 kernels of the decode library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvd {

constexpr int kWave = 64;
constexpr int kBlockTokens = 16;
// Initial running maximum: finite, so max - max never forms inf - inf.
constexpr float kMinusBig = -1.0e30f;
constexpr float kLog2e = 1.4426950408889634f;

// bf16 is the top half of an fp32 word: widening is a shift or a mask.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// a.lo*b.lo + a.hi*b.hi + c with bf16 operands and fp32 accumulation.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Round fp32 to bf16, nearest even (hardware conversion).
__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over the 8 lanes of each half-row (lanes 8k .. 8k+7); every lane of the
// group receives the total.  quad_perm [1,0,3,2] and [2,3,0,1] form the quad
// sums, row_half_mirror adds the other quad of the half-row.
__device__ __forceinline__ float sum_over_8(float x) {
  x += dpp_move<0xB1>(x);
  x += dpp_move<0x4E>(x);
  x += dpp_move<0x141>(x);
  return x;
}

__device__ __forceinline__ float shfl_xor_f(float x, int mask) {
  return __shfl_xor(x, mask, kWave);
}

__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

template <int N> struct Words;
template <> struct Words<1> { typedef uint32_t type; };
template <> struct Words<2> { typedef uint2 type; };
template <> struct Words<4> { typedef uint4 type; };

// Load N consecutive 32-bit words (N = 1, 2 or 4) with one vector load.
template <int N>
__device__ __forceinline__ void load_words(uint32_t* dst, const uint32_t* src) {
  typedef typename Words<N>::type V;
  V v = *reinterpret_cast<const V*>(src);
  if constexpr (N == 1) {
    dst[0] = v;
  } else if constexpr (N == 2) {
    dst[0] = v.x; dst[1] = v.y;
  } else {
    dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
  }
}

template <int N>
__device__ __forceinline__ void store_words(uint32_t* dst, const uint32_t* src) {
  typedef typename Words<N>::type V;
  V v;
  if constexpr (N == 1) {
    v = src[0];
  } else if constexpr (N == 2) {
    v.x = src[0]; v.y = src[1];
  } else {
    v.x = src[0]; v.y = src[1]; v.z = src[2]; v.w = src[3];
  }
  *reinterpret_cast<V*>(dst) = v;
}

}  // namespace kvd
