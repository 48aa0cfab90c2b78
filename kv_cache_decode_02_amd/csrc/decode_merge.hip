// Log-sum-exp merge of split-KV partials into the decode output (the
// combination itself is in kvd_merge.h).  A sequence with no positions gets
// zeros.  Fixed partitions: P_b = ceil(L_b / partition); balanced split: P_b
// is the piece count that the partial kernel recorded.
#include "kvd_device.h"
#include "kvd_internal.h"
#include "kvd_merge.h"

namespace kvd {
namespace {

// WPB wavefronts per (b, h): one (four (b, h) per 256-thread workgroup) when
// a (b, h) has few pieces, four (one (b, h) per workgroup) when it may have
// many; the waves of one (b, h) take every WPB-th run of 64 slots and add
// their sums through LDS.  Rows of the non-empty slots are read kRows at a
// time.
template <bool BF16, int D, int WPB>
__global__ __launch_bounds__(256) void merge_kernel(MergeLaunch a) {
  constexpr int DL = MergeShape<D>::DL, kRows = MergeShape<D>::kRows;
  __shared__ float red[WPB][D + 2];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int sw = wave % WPB;  // this wave's part of the (b, h)
  const int bh = blockIdx.x * (4 / WPB) + wave / WPB;
  if (bh >= a.batch * a.num_q_heads) return;  // with WPB > 1 the whole workgroup
  const int b = bh / a.num_q_heads;

  int len = a.seq_lens[b];
  len = min(len, a.max_blocks_per_seq_tokens);
  const size_t P = a.num_partitions;
  int np = len <= 0 ? 0 : a.counts ? a.counts[bh] : (len + a.partition_tokens - 1) / a.partition_tokens;
  np = min(max(np, 0), static_cast<int>(P));
  const float2* ml = reinterpret_cast<const float2*>(a.ws_ml) + bh * P;
  // (fp16 rows for the latent width: a float pointer to their halves)
  const float* o = a.ws_o + bh * P * (kF16Rows<D> ? D / 2 : D);

  const bool active = lane * DL < D;
  if constexpr (WPB == 1) {
    float acc[DL], den;
    merge_pieces<D>(ml, o, np, lane, acc, den);
    store_merged<BF16, D>(a.out, bh, lane, acc, den);
    return;
  }

  // Pass 1, lanes over slots: the common maximum.  Slots with l = 0 (pieces
  // without valid tokens) carry no weight and are skipped.
  float M = kMinusBig;
  for (int p = sw * kWave + lane; p < np; p += kWave * WPB) {
    const float2 v = ml[p];
    if (v.y > 0.f) M = fmaxf(M, v.x);
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) M = fmaxf(M, shfl_xor_f(M, s));
  if constexpr (WPB > 1) {
    if (lane == 0) red[sw][D] = M;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < WPB; ++w) M = fmaxf(M, red[w][D]);
    __syncthreads();
  }

  // Pass 2: runs of 64 slots; the non-empty ones from a ballot, their weights
  // from the owning lane, their rows kRows at a time.
  float acc[DL];
#pragma unroll
  for (int d = 0; d < DL; ++d) acc[d] = 0.f;
  float den = 0.f;
  for (int p0 = sw * kWave; p0 < np; p0 += kWave * WPB) {
    const float2 v = p0 + lane < np ? ml[p0 + lane] : make_float2(kMinusBig, 0.f);
    const float w_lane = v.y > 0.f ? exp2_fast(v.x - M) : 0.f;
    den += w_lane * v.y;
    const float wr_lane = kF16Rows<D> ? w_lane * v.y : w_lane;  // weight of the lane's row
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
  if constexpr (WPB > 1) {
    if (active) {
#pragma unroll
      for (int d = 0; d < DL; ++d) red[sw][lane * DL + d] = acc[d];
    }
    if (lane == 0) red[sw][D + 1] = den;
    __syncthreads();
    if (sw != 0) return;
    if (active) {
#pragma unroll
      for (int d = 0; d < DL; ++d) {
        float x = acc[d];
#pragma unroll
        for (int w = 1; w < WPB; ++w) x += red[w][lane * DL + d];
        acc[d] = x;
      }
    }
#pragma unroll
    for (int w = 1; w < WPB; ++w) den += red[w][D + 1];
  }
  store_merged<BF16, D>(a.out, bh, lane, acc, den);
}

template <bool BF16, int WPB>
hipError_t launch_merge_waves(const MergeLaunch& a, hipStream_t stream) {
  const long long bh = static_cast<long long>(a.batch) * a.num_q_heads;
  const dim3 grid(static_cast<unsigned>((bh + (4 / WPB) - 1) / (4 / WPB)));
  switch (a.head_dim) {
    case 32: hipLaunchKernelGGL((merge_kernel<BF16, 32, WPB>), grid, dim3(256), 0, stream, a); break;
    case 64: hipLaunchKernelGGL((merge_kernel<BF16, 64, WPB>), grid, dim3(256), 0, stream, a); break;
    case 128: hipLaunchKernelGGL((merge_kernel<BF16, 128, WPB>), grid, dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL((merge_kernel<BF16, 512, WPB>), grid, dim3(256), 0, stream, a); break;
  }
  return hipGetLastError();
}

// Four waves per (b, h) once a (b, h) may hold more than 64 pieces.
template <bool BF16>
hipError_t launch_merge_typed(const MergeLaunch& a, hipStream_t stream) {
  return a.num_partitions > 64 ? launch_merge_waves<BF16, 4>(a, stream)
                               : launch_merge_waves<BF16, 1>(a, stream);
}

}  // namespace

hipError_t launch_merge(const MergeLaunch& a, hipStream_t stream) {
  return a.bf16 ? launch_merge_typed<true>(a, stream) : launch_merge_typed<false>(a, stream);
}

}  // namespace kvd
