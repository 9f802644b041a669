// Outlier feature columns of the LLM.int8() mixed-precision decomposition
// ("Transformers 单 GPU 高效推理：bitsandbytes LLM.int8 …", core idea: feature
// columns holding values beyond the threshold go through fp16):
// flags[k] = (max_m |x[m,k]| >= threshold).
//
//   k_colflag  one workgroup per 16 columns (256 for K = 4096): thread t reads
//              the 16-byte chunk (t & 1) of rows t/2, t/2 + 128, ..., four
//              rows in flight per round of 512 rows; the 128 row groups are
//              combined in LDS and the workgroup writes the 16 flags.
//
// The ascending list of flagged columns and its count are compacted from the
// flags by an extra workgroup of the masked activation quantizer that runs
// next (quant.hip), which saves a launch; the count stays on the device.
#include "q8_device.hpp"
#include "q8_kernels.hpp"

namespace q8 {
namespace {

constexpr int kFlagCols = 16;                  // columns per workgroup: 2 chunks of 8 fp16
constexpr int kFlagThreads = 256;
constexpr int kRowGroups = kFlagThreads / 2;   // 128 rows per load round
constexpr int kRounds = 4;                     // rounds per workgroup (512 rows)
constexpr int kFlagRows = kRowGroups * kRounds;

__global__ __launch_bounds__(kFlagThreads) void k_colflag(const uint16_t* __restrict__ x, int M, int K,
                                                          float threshold, uint8_t* __restrict__ flags) {
  __shared__ float red[kRowGroups][kFlagCols + 1];
  __shared__ float red2[kFlagThreads / kFlagCols][kFlagCols];
  const int tid = threadIdx.x;
  const int c2 = tid & 1, rg = tid >> 1;
  const int col = blockIdx.x * kFlagCols + c2 * 8;       // K is a multiple of 16: always < K
  float mx[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) mx[e] = 0.0f;
  for (int m0 = 0; m0 < M; m0 += kFlagRows) {
    v4i ch[kRounds];
#pragma unroll
    for (int u = 0; u < kRounds; ++u) {
      int m = m0 + u * kRowGroups + rg;
      m = m < M ? m : M - 1;                  // rows past M repeat row M-1: the max is unchanged
      ch[u] = *(const v4i*)(x + (size_t)m * K + col);
    }
#pragma unroll
    for (int u = 0; u < kRounds; ++u) {
      float v[8];
      Chunk<DT_F16>::decode(ch[u], v);
#pragma unroll
      for (int e = 0; e < 8; ++e) mx[e] = fmaxf(mx[e], fabsf(v[e]));
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rg][c2 * 8 + e] = mx[e];
  __syncthreads();
  {
    // 16 parts of 8 row groups for each of the 16 columns
    const int c = tid & 15, part = tid >> 4;
    float v = red[part * 8][c];
#pragma unroll
    for (int g = 1; g < 8; ++g) v = fmaxf(v, red[part * 8 + g][c]);
    red2[part][c] = v;
  }
  __syncthreads();
  if (tid < kFlagCols) {
    float v = red2[0][tid];
#pragma unroll
    for (int p = 1; p < kFlagThreads / kFlagCols; ++p) v = fmaxf(v, red2[p][tid]);
    flags[blockIdx.x * kFlagCols + tid] = v >= threshold ? 1 : 0;
  }
}

}  // namespace

hipError_t launch_outlier_flags(const uint16_t* x_f16, int64_t M, int64_t K, float threshold, uint8_t* flags,
                                hipStream_t st) {
  k_colflag<<<(unsigned)(K / kFlagCols), kFlagThreads, 0, st>>>(x_f16, (int)M, (int)K, threshold, flags);
  return hipGetLastError();
}

}  // namespace q8
