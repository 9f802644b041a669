// Internal launcher of the measurement helper (host side, not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8 {

// ceiling.hip: `workgroups` x 256 threads, each wave iters x 4 MFMAs of the
// kind (0: int8 32x32x32, 2: fp8 32x32x64) on registers; sink[workgroups * 256].
hipError_t launch_mfma_loop(int kind, int64_t iters, int64_t workgroups, int* sink, hipStream_t st);

}  // namespace q8
