// Streaming-read probe: the best sustained HBM read rate of this device, as
// context for the decode kernels, which spend their time reading the cache
// ("KV-Cache——为什么AI回复越来越快", 04: decode is bound by moving the cache,
// not by arithmetic).  Each thread reads 16-byte words with eight loads in
// flight and folds them into one value, which it writes only if it equals a
// sentinel, so the reads cannot be dropped and almost nothing is written.
#include "kvd_device.h"
#include "kvd_internal.h"

namespace kvd {
namespace {

constexpr int kThreads = 256;
constexpr int kGroups = 2048;
constexpr int kUnroll = 8;

// Workgroup g reads the g-th of kGroups contiguous spans of the buffer;
// within a span the threads read consecutive 16-byte words, kUnroll loads in
// flight each.  (Measured on MI355X over 1 GiB: contiguous spans per
// workgroup stream faster than a grid-stride loop, 6.1-6.2 against 5.6 TB/s.)
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* src, size_t n16,
                                                               uint32_t* sink, uint32_t sentinel) {
  const size_t span = (n16 + kGroups - 1) / kGroups;
  const size_t begin = static_cast<size_t>(blockIdx.x) * span;
  const size_t end = begin + span < n16 ? begin + span : n16;
  size_t i = begin + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * kThreads < end; i += kUnroll * kThreads) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = src[i + u * kThreads];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < end; i += kThreads) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == sentinel) sink[static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x] = acc;
}

}  // namespace

int stream_read_groups() { return kGroups; }

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(kGroups), dim3(kThreads), 0, stream,
                     static_cast<const uint4*>(src), bytes / 16, sink, 0x9E3779B9u);
  return hipGetLastError();
}

}  // namespace kvd
