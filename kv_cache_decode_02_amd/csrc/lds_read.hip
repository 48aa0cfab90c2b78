// LDS-read probe: the sustained read rate of one compute unit's LDS for the
// two read kinds the MLA and prefill kernels feed their MFMAs with (16-byte
// reads, and 8-byte transposing reads of 16-bit elements), as context for
// those kernels' step times.  One workgroup of eight waves per compute unit
// reads a 64 KiB LDS array over and over, eight reads in flight per lane,
// every instruction touching consecutive bytes (no bank conflicts), and folds
// what it reads into one value, written only if it equals a sentinel.  Wave
// 0 of every workgroup records the shader clock around its read loop.
#include "kvd_device.h"
#include "kvd_internal.h"
#include "kvd_probe.h"

namespace kvd {
namespace {

constexpr int kThreads = 512;
constexpr int kLdsBytes = 64 * 1024;   // the array that is read
constexpr int kLdsAlloc = 96 * 1024;   // allocated: one workgroup per compute unit
constexpr int kInFlight = 8;

template <int MODE>
__global__ __launch_bounds__(kThreads) void lds_read_kernel(int iters, unsigned long long* cycles,
                                                            uint32_t* sink, uint32_t sentinel) {
  __shared__ __attribute__((aligned(16))) uint4 buf[kLdsAlloc / 16];
  const int tid = threadIdx.x;
  for (int i = tid; i < kLdsBytes / 16; i += kThreads)
    buf[i] = make_uint4(i, i * 3u, i * 5u, i * 7u);
  __syncthreads();
  const int lane = tid & (kWave - 1), wave = tid >> 6;
  // Bytes one instruction of a wave reads, and where a wave starts.
  constexpr int kInst = MODE == 0 ? kWave * 16 : kWave * 8;
  const uint8_t* base = reinterpret_cast<const uint8_t*>(buf);
  uint32_t off = static_cast<uint32_t>(wave * (kLdsBytes / 8) + lane * (kInst / kWave));
  uint32_t acc = 0;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    if constexpr (MODE == 0) {
      uint4 v[kInFlight];
#pragma unroll
      for (int k = 0; k < kInFlight; ++k)
        v[k] = *reinterpret_cast<const uint4*>(base + ((off + k * kInst) & (kLdsBytes - 1)));
#pragma unroll
      for (int k = 0; k < kInFlight; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    } else {
      uint2 v[kInFlight];
#pragma unroll
      for (int k = 0; k < kInFlight; ++k)
        v[k] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_t*)(base + ((off + k * kInst) & (kLdsBytes - 1)))));
#pragma unroll
      for (int k = 0; k < kInFlight; ++k) acc ^= v[k].x ^ v[k].y;
    }
    off = (off + kInFlight * kInst) & (kLdsBytes - 1);
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  if (tid == 0) cycles[blockIdx.x] = t1 - t0;
  if (acc == sentinel) sink[static_cast<size_t>(blockIdx.x) * kThreads + tid] = acc;
}

}  // namespace

int lds_read_threads() { return kThreads; }

int lds_read_bytes_per_lane_iter(int mode) { return kInFlight * (mode == 0 ? 16 : 8); }

hipError_t launch_lds_read(int mode, int groups, int iters, unsigned long long* cycles,
                           uint32_t* sink, hipStream_t stream) {
  if (mode == 0)
    hipLaunchKernelGGL(lds_read_kernel<0>, dim3(groups), dim3(kThreads), 0, stream, iters, cycles,
                       sink, 0x9E3779B9u);
  else
    hipLaunchKernelGGL(lds_read_kernel<1>, dim3(groups), dim3(kThreads), 0, stream, iters, cycles,
                       sink, 0x9E3779B9u);
  return hipGetLastError();
}

}  // namespace kvd
