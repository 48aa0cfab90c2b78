// Launchers of the measurement kernels that are not steps of the decode path
// (the LDS-read probe); the C ABI in api.cpp wraps them.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace kvd {

int lds_read_threads();
int lds_read_bytes_per_lane_iter(int mode);
hipError_t launch_lds_read(int mode, int groups, int iters, unsigned long long* cycles,
                           uint32_t* sink, hipStream_t stream);

}  // namespace kvd
