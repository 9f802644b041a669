// Row-wise quantizers: per-output-channel weights (INT8 asymmetric, FP8 e4m3)
// and per-token activations (INT8 symmetric with the code row-sum, FP8 e4m3
// with the activation-scale upper bound).
//
// Weights (offline, once per model): one 256-thread workgroup per row, IEEE
// division for every code.  Activations (every forward, HBM-bound): one wave
// per row, four rows per 256-thread workgroup, no workgroup barriers; each
// lane keeps its 16-byte chunks of the row in registers so the row is read
// from HBM once, the absmax is a wave reduction, and the codes are emitted
// from the registers.  For 16-bit inputs the quotient x / S comes from two
// FMAs on RN(1/S) (same codes as the division over that whole input domain),
// the integer rounding from adding 1.5 * 2^23, the byte packing from v_perm
// and the code row sum from v_dot4.  Per row: K * sizeof(in) bytes in, K
// bytes + 8 bytes of metadata out.
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

// ---------------------------------------------------------------- one wave per row
constexpr int kRowsPerBlock = kThreads / 64;

// Chunk loads for a row handled by one wave: lane l owns chunks l, l+64, ...
// of which the first CACHE stay in registers.
template <int DT, int CACHE>
struct WaveRow {
  static constexpr int E = Chunk<DT>::kElems;
  v4i cache[CACHE];
  template <class F>
  __device__ __forceinline__ void load(const void* base, int64_t row, int nch, int lane, F&& each) {
#pragma unroll
    for (int j = 0; j < CACHE; ++j) {
      const int c = lane + 64 * j;
      if (c < nch) {
        cache[j] = load_chunk<DT>(base, row, c);
        each(cache[j], c);
      }
    }
    for (int c = lane + 64 * CACHE; c < nch; c += 64) each(load_chunk<DT>(base, row, c), c);
  }
  template <class F>
  __device__ __forceinline__ void replay(const void* base, int64_t row, int nch, int lane, F&& each) {
#pragma unroll
    for (int j = 0; j < CACHE; ++j) {
      const int c = lane + 64 * j;
      if (c < nch) each(cache[j], c);
    }
    for (int c = lane + 64 * CACHE; c < nch; c += 64) each(load_chunk<DT>(base, row, c), c);
  }
};

// ---------------------------------------------------------------- rows -> FP8 e4m3 (weights and activations)
// bound: activation scale upper bound on the row absmax (+inf for none).
template <int DT, int CACHE>
__global__ __launch_bounds__(kThreads) void k_quant_rows_fp8(const void* __restrict__ x, int64_t R, int64_t K,
                                                             float bound, uint8_t* __restrict__ xq,
                                                             float* __restrict__ x_scale) {
  constexpr int E = Chunk<DT>::kElems;
  const int lane = threadIdx.x & 63;
  const int64_t m = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (m >= R) return;                                  // whole wave
  const int nch = (int)(K / E);
  const int64_t row = m * K;
  WaveRow<DT, CACHE> wr;
  float amax = 0.0f;
  wr.load(x, row, nch, lane, [&](const v4i& ch, int) {
    float v[E];
    Chunk<DT>::decode(ch, v);
#pragma unroll
    for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(v[e]));
  });
  amax = wave_max(amax);
  const float a = fminf(amax, bound);
  float s = a / kFp8Max;
  s = s < kEps ? kEps : s;
  const float r = 1.0f / s;
  // the two-FMA quotient is used where the scale comes from a 16-bit row absmax
  const bool fast = (DT != DT_F32) && (amax <= bound);
  wr.replay(x, row, nch, lane, [&](const v4i& ch, int c) {
    float v[E];
    Chunk<DT>::decode(ch, v);
    uint32_t words[E / 4];
#pragma unroll
    for (int g = 0; g < E / 4; ++g) {
      float q[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float xv = v[4 * g + e];
        const float y = fast ? __builtin_copysignf(quot_fma(xv, s, r), xv) : xv / s;
        q[e] = fminf(fmaxf(y, -kFp8Max), kFp8Max);
      }
      words[g] = pack4_e4m3(q[0], q[1], q[2], q[3]);
    }
    store_codes<E>(xq, row + (int64_t)c * E, words);
  });
  if (lane == 0) x_scale[m] = s;
}

// ---------------------------------------------------------------- activations, INT8 sym (+ row sum)
// colflag (nullable, [K] bytes): nonzero marks a column whose values are
// treated as 0 (the outlier columns of the mixed-precision decomposition).
template <int DT, int CACHE>
__global__ __launch_bounds__(kThreads) void k_quant_act_i8(const void* __restrict__ x, int64_t M, int64_t K,
                                                           const uint8_t* __restrict__ colflag,
                                                           int8_t* __restrict__ xq,
                                                           float* __restrict__ x_scale,
                                                           int32_t* __restrict__ x_rowsum) {
  constexpr int E = Chunk<DT>::kElems;
  const int lane = threadIdx.x & 63;
  const int64_t m = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (m >= M) return;                                  // whole wave
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
  WaveRow<DT, CACHE> wr;
  float amax = 0.0f;
  wr.load(x, row, nch, lane, [&](const v4i& ch, int c) {
    float v[E];
    decode_masked(ch, c, v);
#pragma unroll
    for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(v[e]));
  });
  amax = wave_max(amax);
  float s = amax / 127.0f;
  s = s < kEps ? kEps : s;
  const float r = 1.0f / s;
  int qsum = 0;
  // |x / s| <= 127 (s = absmax/127 rounded, or the 1e-8 floor), so the codes
  // need no clamp and the 1.5 * 2^23 rounding applies.
  wr.replay(x, row, nch, lane, [&](const v4i& ch, int c) {
    float v[E];
    decode_masked(ch, c, v);
    uint32_t words[E / 4];
#pragma unroll
    for (int g = 0; g < E / 4; ++g) {
      uint32_t b[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float xv = v[4 * g + e];
        const float y = (DT == DT_F32) ? xv / s : quot_fma(xv, s, r);
        b[e] = rne_int8_bits(y);
      }
      words[g] = pack_lo_bytes(b[0], b[1], b[2], b[3]);
      qsum = sum_i8x4(words[g], qsum);
    }
    store_codes<E>(xq, row + (int64_t)c * E, words);
  });
  qsum = wave_sum(qsum);
  if (lane == 0) {
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
  dim3 grid((unsigned)((R + kRowsPerBlock - 1) / kRowsPerBlock)), block(kThreads);
  const int64_t per_lane = K / (dt == DT_F32 ? 4 : 8) / 64;
  const bool big = per_lane > 8;
  switch (dt) {
    case DT_F32:
      if (big) k_quant_rows_fp8<DT_F32, 32><<<grid, block, 0, st>>>(x, R, K, bound, xq, x_scale);
      else k_quant_rows_fp8<DT_F32, 8><<<grid, block, 0, st>>>(x, R, K, bound, xq, x_scale);
      break;
    case DT_F16:
      if (big) k_quant_rows_fp8<DT_F16, 32><<<grid, block, 0, st>>>(x, R, K, bound, xq, x_scale);
      else k_quant_rows_fp8<DT_F16, 8><<<grid, block, 0, st>>>(x, R, K, bound, xq, x_scale);
      break;
    default:
      if (big) k_quant_rows_fp8<DT_BF16, 32><<<grid, block, 0, st>>>(x, R, K, bound, xq, x_scale);
      else k_quant_rows_fp8<DT_BF16, 8><<<grid, block, 0, st>>>(x, R, K, bound, xq, x_scale);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_quant_act_i8(const void* x, int dt, int64_t M, int64_t K, const uint8_t* colflag,
                               int8_t* xq, float* x_scale, int32_t* x_rowsum, hipStream_t st) {
  dim3 grid((unsigned)((M + kRowsPerBlock - 1) / kRowsPerBlock)), block(kThreads);
  const int64_t per_lane = K / (dt == DT_F32 ? 4 : 8) / 64;
  const bool big = per_lane > 8;
  switch (dt) {
    case DT_F32:
      if (big) k_quant_act_i8<DT_F32, 32><<<grid, block, 0, st>>>(x, M, K, colflag, xq, x_scale, x_rowsum);
      else k_quant_act_i8<DT_F32, 8><<<grid, block, 0, st>>>(x, M, K, colflag, xq, x_scale, x_rowsum);
      break;
    case DT_F16:
      if (big) k_quant_act_i8<DT_F16, 32><<<grid, block, 0, st>>>(x, M, K, colflag, xq, x_scale, x_rowsum);
      else k_quant_act_i8<DT_F16, 8><<<grid, block, 0, st>>>(x, M, K, colflag, xq, x_scale, x_rowsum);
      break;
    default:
      if (big) k_quant_act_i8<DT_BF16, 32><<<grid, block, 0, st>>>(x, M, K, colflag, xq, x_scale, x_rowsum);
      else k_quant_act_i8<DT_BF16, 8><<<grid, block, 0, st>>>(x, M, K, colflag, xq, x_scale, x_rowsum);
      break;
  }
  return hipGetLastError();
}

}  // namespace q8
