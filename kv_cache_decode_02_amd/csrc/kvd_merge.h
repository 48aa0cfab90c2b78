// Log-sum-exp combination of split-KV pieces for one (sequence, head), used by
// the merge kernel.
//
// Piece p carries (m_p, l_p, acc_p) with m_p in log2 units, l_p = sum
// 2^(z' - m_p) and acc_p = sum 2^(z' - m_p) V.  With M = max_p m_p the
// softmax over all positions is
//   out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p,
// the exact regrouping of the stable softmax of "KV缓存原理与显存估算"
// (知识点二: subtracting one common maximum leaves the softmax unchanged).
// Pieces with l = 0 (no valid tokens) carry no weight and are skipped.
#pragma once

#include "kvd_device.h"

namespace kvd {

template <int D>
struct MergeShape {
  static constexpr int DL = D >= kWave ? D / kWave : 1;  // dims per lane
  static constexpr int kRows = 8;                         // rows in flight
};

// The lane's DL consecutive floats of a piece row, as 16-byte (or 8-byte)
// vector loads, or zeros when `take` is false.
template <int DL>
__device__ __forceinline__ void load_row(float (&dst)[DL], const float* src, bool take) {
  if (take) {
    if constexpr (DL % 4 == 0) {
#pragma unroll
      for (int d = 0; d < DL; d += 4) {
        const float4 v = *reinterpret_cast<const float4*>(src + d);
        dst[d] = v.x;
        dst[d + 1] = v.y;
        dst[d + 2] = v.z;
        dst[d + 3] = v.w;
      }
    } else if constexpr (DL == 2) {
      const float2 v = *reinterpret_cast<const float2*>(src);
      dst[0] = v.x;
      dst[1] = v.y;
    } else {
#pragma unroll
      for (int d = 0; d < DL; ++d) dst[d] = src[d];
    }
  } else {
#pragma unroll
    for (int d = 0; d < DL; ++d) dst[d] = 0.f;
  }
}

// Rows of a piece: unnormalised fp32 sums (paged path), or for the latent
// width the sums divided by the piece's weight sum l, in fp16 (MLA path).
template <int D>
constexpr bool kF16Rows = D == 512;

// Row `row` of the pieces at `o` (for fp16 rows `o` addresses halves), the
// lane's DL dims, or zeros without `take`.
template <int D, int DL>
__device__ __forceinline__ void load_piece_row(float (&dst)[DL], const float* o, int row, int lane,
                                               bool take) {
  if constexpr (kF16Rows<D>) {
    static_assert(DL == 8, "fp16 rows: 16 bytes per lane");
    if (take) {
      const uint4 v = *reinterpret_cast<const uint4*>(reinterpret_cast<const _Float16*>(o) +
                                                      static_cast<size_t>(row) * D + lane * DL);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f16x2_t h = __builtin_bit_cast(f16x2_t, w[k]);
        dst[2 * k] = static_cast<float>(h[0]);
        dst[2 * k + 1] = static_cast<float>(h[1]);
      }
    } else {
#pragma unroll
      for (int d = 0; d < DL; ++d) dst[d] = 0.f;
    }
  } else {
    load_row<DL>(dst, o + static_cast<size_t>(row) * D + lane * DL, take);
  }
}

// One wave combines pieces [0, np) of one (b, h): `ml` holds their (m, l)
// pairs and `o` their rows of D floats.  On return lane `lane` holds dims
// lane * DL .. of the unnormalised sum and every lane the denominator.
template <int D>
__device__ __forceinline__ void merge_pieces(const float2* ml, const float* o, int np, int lane,
                                             float (&acc)[MergeShape<D>::DL], float& den) {
  constexpr int DL = MergeShape<D>::DL, kRows = MergeShape<D>::kRows;
  const bool active = lane * DL < D;
#pragma unroll
  for (int d = 0; d < DL; ++d) acc[d] = 0.f;
  if (np <= kRows) {
    // Few pieces: the pairs and the rows in one round trip.
    const float2 v = lane < np ? ml[lane] : make_float2(kMinusBig, 0.f);
    float rows[kRows][DL];
#pragma unroll
    for (int k = 0; k < kRows; ++k) load_piece_row<D, DL>(rows[k], o, k, lane, k < np && active);
    float M = v.y > 0.f ? v.x : kMinusBig;
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) M = fmaxf(M, shfl_xor_f(M, s));
    const float w_lane = v.y > 0.f ? exp2_fast(v.x - M) : 0.f;
    den = w_lane * v.y;
    const float wr_lane = kF16Rows<D> ? w_lane * v.y : w_lane;  // weight of the lane's row
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) den += shfl_xor_f(den, s);
    // (An empty piece, weight 0, may hold no row values at all: it is
    // skipped rather than multiplied by 0.)
#pragma unroll
    for (int k = 0; k < kRows; ++k) {
      const float w = __shfl(wr_lane, k, kWave);
      if (w != 0.f) {
#pragma unroll
        for (int d = 0; d < DL; ++d) acc[d] = fmaf(w, rows[k][d], acc[d]);
      }
    }
    return;
  }
  // Pass 1, lanes over pieces: the common maximum.
  float M = kMinusBig;
  for (int p = lane; p < np; p += kWave) {
    const float2 v = ml[p];
    if (v.y > 0.f) M = fmaxf(M, v.x);
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) M = fmaxf(M, shfl_xor_f(M, s));
  // Pass 2: runs of 64 pieces; the non-empty ones from a ballot, their
  // weights from the owning lane, their rows kRows at a time.
  den = 0.f;
  for (int p0 = 0; p0 < np; p0 += kWave) {
    const float2 v = p0 + lane < np ? ml[p0 + lane] : make_float2(kMinusBig, 0.f);
    const float w_lane = v.y > 0.f ? exp2_fast(v.x - M) : 0.f;
    den += w_lane * v.y;
    const float wr_lane = kF16Rows<D> ? w_lane * v.y : w_lane;
    uint64_t mask = __builtin_amdgcn_ballot_w64(v.y > 0.f);
    while (mask) {
      int idx[kRows];
#pragma unroll
      for (int k = 0; k < kRows; ++k) {
        idx[k] = mask ? static_cast<int>(__builtin_ctzll(mask)) : -1;
        mask &= mask - 1;
      }
      float rows[kRows][DL];
#pragma unroll
      for (int k = 0; k < kRows; ++k)
        load_piece_row<D, DL>(rows[k], o, p0 + max(idx[k], 0), lane, idx[k] >= 0 && active);
#pragma unroll
      for (int k = 0; k < kRows; ++k) {
        const float w = __shfl(wr_lane, idx[k] >= 0 ? idx[k] : 0, kWave);
        if (idx[k] >= 0) {
#pragma unroll
          for (int d = 0; d < DL; ++d) acc[d] = fmaf(w, rows[k][d], acc[d]);
        }
      }
    }
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) den += shfl_xor_f(den, s);
}

// out_row[d] = acc / den for the lane's dims, rounded to the output type (a
// row without positions has den = 0 and gets zeros).
template <bool BF16, int D>
__device__ __forceinline__ void store_merged(void* out, size_t row, int lane,
                                             const float (&acc)[MergeShape<D>::DL], float den) {
  constexpr int DL = MergeShape<D>::DL;
  if (lane * DL >= D) return;
  const float inv = den > 0.f ? 1.0f / den : 0.f;
  if constexpr (BF16) {
    uint16_t* o = static_cast<uint16_t*>(out) + row * D + lane * DL;
#pragma unroll
    for (int d = 0; d < DL; ++d) o[d] = to_bf16_bits(acc[d] * inv);
  } else {
    float* o = static_cast<float*>(out) + row * D + lane * DL;
#pragma unroll
    for (int d = 0; d < DL; ++d) o[d] = acc[d] * inv;
  }
}

}  // namespace kvd
