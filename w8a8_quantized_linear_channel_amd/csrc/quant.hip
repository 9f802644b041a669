// Row-wise quantizers: per-output-channel weights (INT8 asymmetric, FP8 e4m3)
// and per-token activations (INT8 symmetric with the code row-sum, FP8 e4m3
// with the activation-scale upper bound).
//
// One 256-thread workgroup per row.  Each thread reads 16-byte chunks
// (coalesced across the workgroup), keeps up to kCache chunks in registers
// so the row is read from HBM once, reduces min/max/absmax with wave
// shuffles + LDS, then emits codes from the registers.  HBM-bound: per row it
// moves K*sizeof(in) bytes in and K bytes (+ 8 B of metadata) out.
#include "q8_device.hpp"
#include "q8_kernels.hpp"

namespace q8 {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kCache = 8;   // chunks held per thread: rows up to 8*256*8 16-bit values

template <int DT>
__device__ __forceinline__ v4i load_chunk(const void* base, int64_t row_elems_off, int c) {
  constexpr int E = Chunk<DT>::kElems;
  const char* p = (const char*)base;
  constexpr int esz = (DT == DT_F32) ? 4 : 2;
  return *(const v4i*)(p + (row_elems_off + (int64_t)c * E) * esz);
}

// Store E codes (E = 4 or 8) packed in bytes at out + off.
template <int E>
__device__ __forceinline__ void store_codes(void* out, int64_t off, const uint32_t* w);
template <>
__device__ __forceinline__ void store_codes<4>(void* out, int64_t off, const uint32_t* w) {
  *(uint32_t*)((char*)out + off) = w[0];
}
template <>
__device__ __forceinline__ void store_codes<8>(void* out, int64_t off, const uint32_t* w) {
  v2i v = {(int)w[0], (int)w[1]};
  *(v2i*)((char*)out + off) = v;
}

// ---------------------------------------------------------------- weights, INT8 asym
template <int DT>
__global__ __launch_bounds__(kThreads) void k_quant_weight_i8(const void* __restrict__ w, int64_t K,
                                                              int8_t* __restrict__ wq,
                                                              float* __restrict__ w_scale,
                                                              float* __restrict__ w_zp) {
  constexpr int E = Chunk<DT>::kElems;
  __shared__ float red[kWaves];
  const int64_t n = blockIdx.x;
  const int tid = threadIdx.x;
  const int nch = (int)(K / E);
  const int64_t row = n * K;

  v4i cache[kCache];
  float lo = 0.0f, hi = 0.0f;   // the range always contains 0
#pragma unroll
  for (int j = 0; j < kCache; ++j) {
    const int c = tid + j * kThreads;
    if (c < nch) {
      cache[j] = load_chunk<DT>(w, row, c);
      float v[E];
      Chunk<DT>::decode(cache[j], v);
#pragma unroll
      for (int e = 0; e < E; ++e) { lo = fminf(lo, v[e]); hi = fmaxf(hi, v[e]); }
    }
  }
  for (int c = tid + kCache * kThreads; c < nch; c += kThreads) {
    float v[E];
    Chunk<DT>::decode(load_chunk<DT>(w, row, c), v);
#pragma unroll
    for (int e = 0; e < E; ++e) { lo = fminf(lo, v[e]); hi = fmaxf(hi, v[e]); }
  }
  lo = block_min<kWaves>(lo, red);
  hi = block_max<kWaves>(hi, red);

  float s = (hi - lo) / 255.0f;
  s = s < kEps ? kEps : s;
  const float z = -128.0f - __builtin_rintf(lo / s);

  auto emit = [&](const v4i& ch, int c) {
    float v[E];
    Chunk<DT>::decode(ch, v);
    uint32_t words[E / 4];
#pragma unroll
    for (int g = 0; g < E / 4; ++g) {
      int q[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float t = __builtin_rintf(v[4 * g + e] / s) + z;
        t = fminf(fmaxf(t, -128.0f), 127.0f);
        q[e] = (int)t;
      }
      words[g] = pack4_i8(q[0], q[1], q[2], q[3]);
    }
    store_codes<E>(wq, row + (int64_t)c * E, words);
  };
#pragma unroll
  for (int j = 0; j < kCache; ++j) {
    const int c = tid + j * kThreads;
    if (c < nch) emit(cache[j], c);
  }
  for (int c = tid + kCache * kThreads; c < nch; c += kThreads) emit(load_chunk<DT>(w, row, c), c);

  if (tid == 0) { w_scale[n] = s; w_zp[n] = z; }
}

// ---------------------------------------------------------------- rows -> FP8 e4m3 (weights and activations)
template <int DT>
__global__ __launch_bounds__(kThreads) void k_quant_rows_fp8(const void* __restrict__ x, int64_t K,
                                                             float bound, uint8_t* __restrict__ xq,
                                                             float* __restrict__ x_scale) {
  constexpr int E = Chunk<DT>::kElems;
  __shared__ float red[kWaves];
  const int64_t m = blockIdx.x;
  const int tid = threadIdx.x;
  const int nch = (int)(K / E);
  const int64_t row = m * K;

  v4i cache[kCache];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < kCache; ++j) {
    const int c = tid + j * kThreads;
    if (c < nch) {
      cache[j] = load_chunk<DT>(x, row, c);
      float v[E];
      Chunk<DT>::decode(cache[j], v);
#pragma unroll
      for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(v[e]));
    }
  }
  for (int c = tid + kCache * kThreads; c < nch; c += kThreads) {
    float v[E];
    Chunk<DT>::decode(load_chunk<DT>(x, row, c), v);
#pragma unroll
    for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(v[e]));
  }
  amax = block_max<kWaves>(amax, red);
  amax = fminf(amax, bound);            // bound = +inf when there is none
  float s = amax / kFp8Max;
  s = s < kEps ? kEps : s;

  auto emit = [&](const v4i& ch, int c) {
    float v[E];
    Chunk<DT>::decode(ch, v);
    uint32_t words[E / 4];
#pragma unroll
    for (int g = 0; g < E / 4; ++g) {
      float r[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = fminf(fmaxf(v[4 * g + e] / s, -kFp8Max), kFp8Max);
      words[g] = pack4_e4m3(r[0], r[1], r[2], r[3]);
    }
    store_codes<E>(xq, row + (int64_t)c * E, words);
  };
#pragma unroll
  for (int j = 0; j < kCache; ++j) {
    const int c = tid + j * kThreads;
    if (c < nch) emit(cache[j], c);
  }
  for (int c = tid + kCache * kThreads; c < nch; c += kThreads) emit(load_chunk<DT>(x, row, c), c);

  if (tid == 0) x_scale[m] = s;
}

// ---------------------------------------------------------------- activations, INT8 sym (+ row sum)
// colflag (nullable, [K] bytes): nonzero marks a column whose values are
// treated as 0 (the outlier columns of the mixed-precision decomposition).
template <int DT>
__global__ __launch_bounds__(kThreads) void k_quant_act_i8(const void* __restrict__ x, int64_t K,
                                                           const uint8_t* __restrict__ colflag,
                                                           int8_t* __restrict__ xq,
                                                           float* __restrict__ x_scale,
                                                           int32_t* __restrict__ x_rowsum) {
  constexpr int E = Chunk<DT>::kElems;
  __shared__ float red[kWaves];
  __shared__ int redi[kWaves];
  const int64_t m = blockIdx.x;
  const int tid = threadIdx.x;
  const int nch = (int)(K / E);
  const int64_t row = m * K;

  auto decode_masked = [&](const v4i& ch, int c, float* v) {
    Chunk<DT>::decode(ch, v);
    if (colflag != nullptr) {
      const uint8_t* f = colflag + (int64_t)c * E;
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (f[e]) v[e] = 0.0f;
    }
  };

  v4i cache[kCache];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < kCache; ++j) {
    const int c = tid + j * kThreads;
    if (c < nch) {
      cache[j] = load_chunk<DT>(x, row, c);
      float v[E];
      decode_masked(cache[j], c, v);
#pragma unroll
      for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(v[e]));
    }
  }
  for (int c = tid + kCache * kThreads; c < nch; c += kThreads) {
    float v[E];
    decode_masked(load_chunk<DT>(x, row, c), c, v);
#pragma unroll
    for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(v[e]));
  }
  amax = block_max<kWaves>(amax, red);
  float s = amax / 127.0f;
  s = s < kEps ? kEps : s;

  int qsum = 0;
  auto emit = [&](const v4i& ch, int c) {
    float v[E];
    decode_masked(ch, c, v);
    uint32_t words[E / 4];
#pragma unroll
    for (int g = 0; g < E / 4; ++g) {
      int q[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        q[e] = code_sym_i8(v[4 * g + e], s);
        qsum += q[e];
      }
      words[g] = pack4_i8(q[0], q[1], q[2], q[3]);
    }
    store_codes<E>(xq, row + (int64_t)c * E, words);
  };
#pragma unroll
  for (int j = 0; j < kCache; ++j) {
    const int c = tid + j * kThreads;
    if (c < nch) emit(cache[j], c);
  }
  for (int c = tid + kCache * kThreads; c < nch; c += kThreads) emit(load_chunk<DT>(x, row, c), c);

  qsum = block_sum<kWaves>(qsum, redi);
  if (tid == 0) {
    x_scale[m] = s;
    if (x_rowsum) x_rowsum[m] = qsum;
  }
}

}  // namespace

hipError_t launch_quant_weight_i8(const void* w, int dt, int64_t N, int64_t K, int8_t* wq,
                                  float* w_scale, float* w_zp, hipStream_t st) {
  dim3 grid((unsigned)N), block(kThreads);
  switch (dt) {
    case DT_F32: k_quant_weight_i8<DT_F32><<<grid, block, 0, st>>>(w, K, wq, w_scale, w_zp); break;
    case DT_F16: k_quant_weight_i8<DT_F16><<<grid, block, 0, st>>>(w, K, wq, w_scale, w_zp); break;
    default: k_quant_weight_i8<DT_BF16><<<grid, block, 0, st>>>(w, K, wq, w_scale, w_zp); break;
  }
  return hipGetLastError();
}

hipError_t launch_quant_rows_fp8(const void* x, int dt, int64_t R, int64_t K, float bound,
                                 uint8_t* xq, float* x_scale, hipStream_t st) {
  dim3 grid((unsigned)R), block(kThreads);
  switch (dt) {
    case DT_F32: k_quant_rows_fp8<DT_F32><<<grid, block, 0, st>>>(x, K, bound, xq, x_scale); break;
    case DT_F16: k_quant_rows_fp8<DT_F16><<<grid, block, 0, st>>>(x, K, bound, xq, x_scale); break;
    default: k_quant_rows_fp8<DT_BF16><<<grid, block, 0, st>>>(x, K, bound, xq, x_scale); break;
  }
  return hipGetLastError();
}

hipError_t launch_quant_act_i8(const void* x, int dt, int64_t M, int64_t K, const uint8_t* colflag,
                               int8_t* xq, float* x_scale, int32_t* x_rowsum, hipStream_t st) {
  dim3 grid((unsigned)M), block(kThreads);
  switch (dt) {
    case DT_F32: k_quant_act_i8<DT_F32><<<grid, block, 0, st>>>(x, K, colflag, xq, x_scale, x_rowsum); break;
    case DT_F16: k_quant_act_i8<DT_F16><<<grid, block, 0, st>>>(x, K, colflag, xq, x_scale, x_rowsum); break;
    default: k_quant_act_i8<DT_BF16><<<grid, block, 0, st>>>(x, K, colflag, xq, x_scale, x_rowsum); break;
  }
  return hipGetLastError();
}

}  // namespace q8
