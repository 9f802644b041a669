// Outlier feature columns of the LLM.int8() mixed-precision decomposition
// ("Transformers 单 GPU 高效推理：bitsandbytes LLM.int8 …", core idea: feature
// columns holding values beyond the threshold go through fp16):
// flags[k] = (max_m |x[m,k]| >= threshold).
//
//   k_colflag  one workgroup per 64 columns (64 for K = 4096): eight lanes
//              read one row's 128 contiguous bytes of them, so every load
//              is a whole 128-byte line; the 32 row groups of a workgroup
//              take rows rg, rg + 32, ... four at a time, are combined in
//              LDS, and the workgroup writes its 64 flags (a ragged last
//              group of 16-column chunks is masked).
//
// The ascending list of flagged columns and its count are compacted from the
// flags by an extra workgroup of the masked activation quantizer that runs
// next (quant.hip), which saves a launch; the count stays on the device.
#include "q8_device.hpp"
#include "q8_kernels.hpp"

namespace q8 {
namespace {

constexpr int kFlagCols = 64;                  // columns per workgroup: 8 chunks of 8 fp16
constexpr int kFlagThreads = 256;
constexpr int kLanesPerRow = kFlagCols / 8;    // 8
constexpr int kRowGroups = kFlagThreads / kLanesPerRow;   // 32 rows per load round
constexpr int kRounds = 4;                     // loads in flight per thread
constexpr int kFlagRows = kRowGroups * kRounds;

__global__ __launch_bounds__(kFlagThreads) void k_colflag(const uint16_t* __restrict__ x, int M, int K,
                                                          float threshold, uint8_t* __restrict__ flags) {
  __shared__ float red[kRowGroups][kFlagCols + 1];
  const int tid = threadIdx.x;
  const int ch = tid % kLanesPerRow, rg = tid / kLanesPerRow;
  // K is a multiple of 16: a chunk of 8 columns lies wholly inside or past K
  int col = blockIdx.x * kFlagCols + ch * 8;
  const bool inside = col < K;
  col = inside ? col : K - 8;                   // re-reads the last chunk; its flags are not written
  float mx[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) mx[e] = 0.0f;
  for (int m0 = 0; m0 < M; m0 += kFlagRows) {
    v4i c4[kRounds];
#pragma unroll
    for (int u = 0; u < kRounds; ++u) {
      int m = m0 + u * kRowGroups + rg;
      m = m < M ? m : M - 1;                  // rows past M repeat row M-1: the max is unchanged
      c4[u] = *(const v4i*)(x + (size_t)m * K + col);
    }
#pragma unroll
    for (int u = 0; u < kRounds; ++u) {
      float v[8];
      Chunk<DT_F16>::decode(c4[u], v);
#pragma unroll
      for (int e = 0; e < 8; ++e) mx[e] = fmaxf(mx[e], fabsf(v[e]));
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rg][ch * 8 + e] = mx[e];
  __syncthreads();
  if (tid < kFlagCols) {
    float v = red[0][tid];
#pragma unroll
    for (int g = 1; g < kRowGroups; ++g) v = fmaxf(v, red[g][tid]);
    const int k = blockIdx.x * kFlagCols + tid;
    if (k < K) flags[k] = v >= threshold ? 1 : 0;
  }
}

}  // namespace

hipError_t launch_outlier_flags(const uint16_t* x_f16, int64_t M, int64_t K, float threshold, uint8_t* flags,
                                hipStream_t st) {
  k_colflag<<<(unsigned)((K + kFlagCols - 1) / kFlagCols), kFlagThreads, 0, st>>>(x_f16, (int)M, (int)K, threshold,
                                                                                  flags);
  return hipGetLastError();
}

}  // namespace q8
