// Outlier feature columns of the LLM.int8() mixed-precision decomposition:
// O = { k : max_m |x[m,k]| >= threshold }, in ascending order, with |O| kept
// on the device (no host synchronization).
//
//   k_colmax_partial  grid (ceil(K / 2048), ceil(M / 64)): each thread owns 8
//                     adjacent columns (one 16-byte fp16 chunk per row, so a
//                     wave reads 1 KB contiguous per row) and 64 rows, and
//                     writes their partial |x| maxima to partial[row_block][k].
//   k_outlier_select  one workgroup of 1024 threads: each thread owns a run of
//                     adjacent columns, reduces their partial maxima,
//                     compares with the threshold, and a workgroup prefix sum
//                     of the per-thread counts gives every flagged column its
//                     ascending position.  Writes flags[K] (consumed by the
//                     masked activation quantizer), idx[] and the count.
#include "q8_device.hpp"
#include "q8_kernels.hpp"

namespace q8 {
namespace {

constexpr int kColThreads = 256;
constexpr int kSelThreads = 1024;

__global__ __launch_bounds__(kColThreads) void k_colmax_partial(const uint16_t* __restrict__ x, int64_t M,
                                                                int64_t K, float* __restrict__ partial) {
  const int64_t c0 = ((int64_t)blockIdx.x * kColThreads + threadIdx.x) * 8;
  if (c0 >= K) return;
  const int64_t r0 = (int64_t)blockIdx.y * kColmaxRows;
  const int64_t r1 = (r0 + kColmaxRows) < M ? (r0 + kColmaxRows) : M;
  float mx[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) mx[e] = 0.0f;
  for (int64_t r = r0; r < r1; ++r) {
    float v[8];
    Chunk<DT_F16>::decode(*(const v4i*)(x + r * K + c0), v);
#pragma unroll
    for (int e = 0; e < 8; ++e) mx[e] = fmaxf(mx[e], fabsf(v[e]));
  }
  float* out = partial + (int64_t)blockIdx.y * K + c0;
  *(v4f*)out = v4f{mx[0], mx[1], mx[2], mx[3]};
  *(v4f*)(out + 4) = v4f{mx[4], mx[5], mx[6], mx[7]};
}

__global__ __launch_bounds__(kSelThreads) void k_outlier_select(const float* __restrict__ partial, int nparts,
                                                                 int64_t K, float threshold,
                                                                 uint8_t* __restrict__ flags,
                                                                 int32_t* __restrict__ idx,
                                                                 int32_t* __restrict__ cnt,
                                                                 int32_t* __restrict__ user_idx,
                                                                 int32_t* __restrict__ user_cnt) {
  __shared__ int wave_tot[kSelThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool on = threshold > 0.0f;
  const int64_t per = (K + kSelThreads - 1) / kSelThreads;
  const int64_t c0 = (int64_t)tid * per;
  const int64_t c1 = (c0 + per) < K ? (c0 + per) : K;

  int mine = 0;
  for (int64_t k = c0; k < c1; ++k) {
    bool f = false;
    if (on) {
      float c = 0.0f;
      for (int p = 0; p < nparts; ++p) c = fmaxf(c, partial[(int64_t)p * K + k]);
      f = c >= threshold;
    }
    flags[k] = f ? 1 : 0;
    mine += f ? 1 : 0;
  }

  // inclusive scan of `mine` over the workgroup
  int incl = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wave_tot[w];
  int pos = before + incl - mine;

  for (int64_t k = c0; k < c1; ++k) {
    if (flags[k]) {
      idx[pos] = (int32_t)k;
      if (user_idx) user_idx[pos] = (int32_t)k;
      ++pos;
    }
  }
  if (tid == kSelThreads - 1) {
    const int total = before + incl;
    *cnt = total;
    if (user_cnt) *user_cnt = total;
  }
}

}  // namespace

hipError_t launch_outlier_detect(const uint16_t* x_f16, int64_t M, int64_t K, float threshold,
                                 float* partial, uint8_t* flags, int32_t* idx, int32_t* cnt,
                                 int32_t* user_idx, int32_t* user_cnt, hipStream_t st) {
  const int nparts = (int)((M + kColmaxRows - 1) / kColmaxRows);
  if (threshold > 0.0f) {
    dim3 grid((unsigned)((K + 8 * kColThreads - 1) / (8 * kColThreads)), (unsigned)nparts);
    k_colmax_partial<<<grid, kColThreads, 0, st>>>(x_f16, M, K, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  k_outlier_select<<<1, kSelThreads, 0, st>>>(partial, nparts, K, threshold, flags, idx, cnt, user_idx,
                                               user_cnt);
  return hipGetLastError();
}

}  // namespace q8
