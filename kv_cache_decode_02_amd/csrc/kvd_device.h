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

// Pack two fp32 values into one bf16x2 word (round to nearest even); a goes
// to the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// Interleave the bf16 halves of two words: (x.lo, y.lo) and (x.hi, y.hi).
__device__ __forceinline__ uint32_t pair_lo(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x07060302u);
}

constexpr uint32_t kBf16OnePair = 0x3F803F80u;  // (1.0, 1.0) in bf16

typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;

// a.lo*b.lo + a.hi*b.hi + c with fp16 operands and fp32 accumulation.
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c,
                                false);
}

// Two fp32 values as one fp16x2 word, round to nearest even; a to the low half.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  f16x2_t v = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// Two integer-valued fp32 values of magnitude <= 2048 as fp16x2 (exact, so
// the truncating conversion is as good as any).
__device__ __forceinline__ uint32_t pack_f16x2_int(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

constexpr uint32_t kF16OnePair = 0x3C003C00u;  // (1.0, 1.0) in fp16

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

// MFMA operand and result vectors.
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// Eight bf16 values from four 32-bit words (whole-vector bit cast: building
// the vector element by element gave wrong operands on this compiler).
__device__ __forceinline__ bf16x8_t as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  uint4 u = make_uint4(a, b, c, d);
  return __builtin_bit_cast(bf16x8_t, u);
}

// Combine a value over the four 16-lane rows of the wave (lanes l, l ^ 16,
// l ^ 32, l ^ 48).  Each swap returns the lane's own value and the value of
// its partner row, so the combination is the same in every lane.
__device__ __forceinline__ float row_max4(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float row_sum4(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

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


// Raw buffer access.  A buffer resource (base, byte count) lives in scalar
// registers; a load whose byte offset falls at or past the count returns
// zeros instead of touching memory.  The resource word-3 value selects 32-bit
// raw addressing on CDNA (gfx9 family).
typedef __amdgpu_buffer_rsrc_t BufRsrc;
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ BufRsrc make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes,
                                           kRsrcWord3);
}

// Load N consecutive 32-bit words (N = 1, 2 or 4) at byte offset `off`.
template <int N>
__device__ __forceinline__ void buffer_load_words(uint32_t* dst, BufRsrc r, uint32_t off) {
  if constexpr (N == 1) {
    dst[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  } else if constexpr (N == 2) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    dst[0] = v[0]; dst[1] = v[1];
  } else {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    dst[0] = v[0]; dst[1] = v[1]; dst[2] = v[2]; dst[3] = v[3];
  }
}

}  // namespace kvd
