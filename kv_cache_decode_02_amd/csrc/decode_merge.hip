// Log-sum-exp merge of split-KV partials into the decode output.
//
// For one (b, h) the partitions p = 0 .. P_b - 1 carry (m_p, l_p, acc_p) with
// m_p in log2 units, l_p = sum 2^(z' - m_p) and acc_p = sum 2^(z' - m_p) V.
// With M = max_p m_p the softmax over all positions is
//   out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p,
// the exact regrouping of the stable softmax of "KV缓存原理与显存估算"
// (知识点二: subtracting one common maximum leaves the softmax unchanged).
// A sequence with no positions gets zeros.
#include "kvd_device.h"
#include "kvd_internal.h"

namespace kvd {
namespace {

template <bool BF16, int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeLaunch a) {
  constexpr int DL = D >= kWave ? D / kWave : 1;  // dims per lane
  const int lane = threadIdx.x & (kWave - 1);
  const int bh = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (bh >= a.batch * a.num_q_heads) return;
  const int b = bh / a.num_q_heads;

  int len = a.seq_lens[b];
  len = min(len, a.max_blocks_per_seq_tokens);
  const int np = len > 0 ? (len + a.partition_tokens - 1) / a.partition_tokens : 0;
  const size_t P = a.num_partitions;
  const float2* ml = reinterpret_cast<const float2*>(a.ws_ml) + bh * P;
  const float* o = a.ws_o + bh * P * D;

  float M = kMinusBig;
  for (int p = lane; p < np; p += kWave) M = fmaxf(M, ml[p].x);
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) M = fmaxf(M, shfl_xor_f(M, s));

  const bool active = lane * DL < D;
  float acc[DL];
#pragma unroll
  for (int d = 0; d < DL; ++d) acc[d] = 0.f;
  float den = 0.f;
#pragma unroll 4
  for (int p = 0; p < np; ++p) {
    const float2 v = ml[p];
    const float w = exp2_fast(v.x - M);
    den = fmaf(w, v.y, den);
    if (active) {
#pragma unroll
      for (int d = 0; d < DL; ++d) acc[d] = fmaf(w, o[p * D + lane * DL + d], acc[d]);
    }
  }
  const float inv = den > 0.f ? 1.0f / den : 0.f;
  if (active) {
    if constexpr (BF16) {
      uint16_t* out = static_cast<uint16_t*>(a.out) + bh * D + lane * DL;
#pragma unroll
      for (int d = 0; d < DL; ++d) out[d] = to_bf16_bits(acc[d] * inv);
    } else {
      float* out = static_cast<float*>(a.out) + bh * D + lane * DL;
#pragma unroll
      for (int d = 0; d < DL; ++d) out[d] = acc[d] * inv;
    }
  }
}

template <bool BF16>
hipError_t launch_merge_typed(const MergeLaunch& a, hipStream_t stream) {
  const long long bh = static_cast<long long>(a.batch) * a.num_q_heads;
  const dim3 grid(static_cast<unsigned>((bh + 3) / 4));
  switch (a.head_dim) {
    case 32: hipLaunchKernelGGL((merge_kernel<BF16, 32>), grid, dim3(256), 0, stream, a); break;
    case 64: hipLaunchKernelGGL((merge_kernel<BF16, 64>), grid, dim3(256), 0, stream, a); break;
    case 128: hipLaunchKernelGGL((merge_kernel<BF16, 128>), grid, dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL((merge_kernel<BF16, 512>), grid, dim3(256), 0, stream, a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeLaunch& a, hipStream_t stream) {
  return a.bf16 ? launch_merge_typed<true>(a, stream) : launch_merge_typed<false>(a, stream);
}

}  // namespace kvd
