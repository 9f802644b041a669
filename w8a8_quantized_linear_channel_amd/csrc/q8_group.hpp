// Internal launchers of the per-group weight path (host side, not part of the
// C ABI).  Weights are INT8 asymmetric per group of `group` consecutive
// columns of a row (group 64 or 128, K a multiple of it); the scales and zero
// points are group-major, [K / group, N], and so are the activation code sums
// per group, [K / group, M].
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8 {

// group.hip
hipError_t launch_quant_weight_grouped(const void* w, int dt, int64_t N, int64_t K, int64_t group, int8_t* wq,
                                       float* w_scale, float* w_zp, hipStream_t st);
// gemv.hip: decode up to kGemvFusedMaxM tokens in one launch, the activation
// quantization fused in (no workspace).
hipError_t launch_gemv_i8_grouped(const void* x, int xdt, int64_t M, int64_t K, const int8_t* wq,
                                  const float* w_scale, const float* w_zp, int64_t group, int64_t N,
                                  const float* bias, void* y, int ydt, hipStream_t st);
// Decode-sized M (<= kGroupGemvMaxM) on codes, scales and group code sums.
hipError_t launch_gemv_group(const int8_t* xq, const float* x_scale, const int32_t* gsum, int64_t M, int64_t K,
                             const int8_t* wq, const float* w_scale, const float* w_zp, int64_t group, int64_t N,
                             const float* bias, void* y, int ydt, hipStream_t st);
hipError_t launch_gemm_group(const int8_t* xq, const float* x_scale, const int32_t* gsum, int64_t M, int64_t K,
                             const int8_t* wq, const float* w_scale, const float* w_zp, int64_t group, int64_t N,
                             const float* bias, void* y, int ydt, hipStream_t st);
constexpr int64_t kGroupGemvMaxM = 16;

// quant.hip: per-token INT8 codes and scales, and the code sum of every group
// of `group` columns of every row, gsum[j * M + m].
hipError_t launch_quant_act_i8_groups(const void* x, int dt, int64_t M, int64_t K, int64_t group, int8_t* xq,
                                      float* x_scale, int32_t* gsum, hipStream_t st);

}  // namespace q8
