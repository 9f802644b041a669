// Internal launcher of the measurement helper (host side, not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8 {

// ceiling.hip: `workgroups` x 256 threads, each wave iters x 4 MFMAs of the
// kind (0: int8 32x32x32, 2: fp8 32x32x64) on registers; sink[workgroups * 256].
hipError_t launch_mfma_loop(int kind, int64_t iters, int64_t workgroups, int* sink, hipStream_t st);
// ceiling.hip: a streaming read of `bytes` (a multiple of 16, < 2^31) by
// `workgroups` x 256 threads; sink[workgroups * 256].
hipError_t launch_stream_read(const void* src, int64_t bytes, int64_t workgroups, int* sink, hipStream_t st);
// ceiling.hip: `count` problems, one wave each, d = c + a . b^T through one
// FP8 MFMA (a, b: [count, 32, 64] e4m3; c, d: [count, 32, 32] fp32).
hipError_t launch_probe_fp8_mfma(const uint8_t* a, const uint8_t* b, const float* c, float* d, int64_t count,
                                 hipStream_t st);

}  // namespace q8
