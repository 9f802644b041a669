// Row-wise quantizers: per-output-channel weights (INT8 asymmetric, FP8 e4m3)
// and per-token activations (INT8 symmetric with the code row-sum, FP8 e4m3
// with the activation-scale upper bound).
//
// One 256-thread workgroup per row.  Each thread keeps its 16-byte chunks of
// the row (chunks tid, tid + 256, ...) in registers, so the row is read from
// HBM once; the absmax (or min/max) is a DPP wave reduction plus four LDS
// slots, and the codes are emitted from the registers, 8 or 4 bytes per
// chunk, consecutive threads writing consecutive bytes.  Many short
// workgroups per CU keep enough loads in flight to approach HBM bandwidth
// even when there are few rows.  Weights (offline) use IEEE division for
// every code.  Activations: for 16-bit inputs the quotient x / S comes from
// two FMAs on RN(1/S) (same codes as the division over that whole input
// domain), the integer rounding from adding 1.5 * 2^23, the byte packing from
// v_perm and the code row sum from v_dot4.  Per row: K * sizeof(in) bytes in,
// K bytes + 8 bytes of metadata out.
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

// ---------------------------------------------------------------- rows (activations; FP8 weights)
enum RowMode : int {
  RM_I8 = 0,         // INT8 symmetric, S = absmax / 127, code row sums
  RM_I8_OUTLIER = 1, // as RM_I8 (fp16 only) with the flagged outlier columns read as 0
  RM_FP8 = 2,        // e4m3, S = min(absmax, bound) / 448
  RM_I8_STATIC = 3,  // INT8 symmetric with a given scale S = bound, codes clamped to +-127
  RM_I8_GROUPS = 4,  // as RM_I8, plus the code sum of every group of glanes consecutive chunks
};
constexpr int kRowCache = 8;   // chunks per thread held in registers: 16-bit rows up to 16384 values
// Rows of up to 2 kThreads chunks (16-bit rows of up to 4096 values) use a
// cache of two chunks: ~50 instead of ~86 registers, so eight row workgroups
// fit on a CU instead of five and a 2048-row activation runs in one round.
constexpr int kSmallCache = 2;

// RM_I8_OUTLIER: the outlier columns (flags[k] != 0) are left out of the row
// absmax and get code 0 (their product goes through the fp16 outlier flow);
// each chunk's 8 flag bytes are one 8-byte load issued with the chunk, and
// chunks that no lane of the wave flags skip the masking.  One extra
// workgroup (the last) compacts the flags into the ascending list of outlier
// columns and its count (for the GEMM's outlier flow and the caller) while
// the others quantize; flags == NULL means no outlier columns.  When
// pan.x_panel is set, the first workgroups of the grid write the panels of
// the first kPanelCols outlier columns, 16 rows each (one value per thread,
// so that the scattered reads spread over many CUs): ceil(R / 16) for X, then
// ceil(N / 16) for the weights; each finds those columns with the same scan
// of the flags.
// At least 4 waves per SIMD (<= 128 VGPRs): several rows per CU keep loads in flight.
template <int MODE, int DT, int CACHE = kRowCache>
__global__ __launch_bounds__(kThreads, 4) void k_quant_rows(
    const void* __restrict__ x, int64_t R, int64_t K, const uint8_t* __restrict__ flags, float bound,
    uint8_t* __restrict__ xq, float* __restrict__ x_scale, int32_t* __restrict__ x_rowsum,
    int32_t* __restrict__ idx, int32_t* __restrict__ cnt, int32_t* __restrict__ user_idx,
    int32_t* __restrict__ user_cnt, int32_t* __restrict__ gsum, int glanes, const OutlierPanels pan) {
  constexpr int E = Chunk<DT>::kElems;
  __shared__ float redf[kWaves];
  __shared__ int redi[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  int64_t bid = blockIdx.x;
  if constexpr (MODE == RM_I8_OUTLIER) {
    constexpr int kPanelRows = kThreads / kPanelCols;
    const int64_t nxp = pan.x_panel != nullptr ? (R + kPanelRows - 1) / kPanelRows : 0;
    const int64_t npan = pan.x_panel != nullptr ? nxp + (pan.N + kPanelRows - 1) / kPanelRows : 0;
    if (bid < npan || bid == npan + R) {
      // Thread t owns the run [c0, c0 + per) of 16-byte flag blocks (K is a
      // multiple of 16); a block prefix sum of the runs' counts gives every
      // flagged column its rank in ascending order.
      const int per = 16 * (int)((K + 16 * kThreads - 1) / (16 * kThreads));
      const int c0 = tid * per;
      int mine = 0, before = 0, total = 0;
      if (flags != nullptr) {
        for (int c = c0; c < c0 + per && c < (int)K; c += 16) {
          const v4i f = *(const v4i*)(flags + c);
#pragma unroll
          for (int i = 0; i < 4; ++i) mine = sum_i8x4((uint32_t)f[i], mine);   // bytes are 0 or 1
        }
        const int incl = wave_incl_scan(mine);
        if (lane == 63) redi[wave] = incl;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          if (w < wave) before += redi[w];
          total += redi[w];
        }
        before += incl - mine;
      }
      // this thread's flagged columns, ascending, with their ranks
      auto each_flagged = [&](auto fn) {
        int pos = before;
        for (int c = c0; c < c0 + per && c < (int)K; c += 16) {
          const v4i f = *(const v4i*)(flags + c);
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (((uint32_t)f[e >> 2] >> (8 * (e & 3))) & 0xffu) fn(pos++, c + e);
        }
      };
      if (bid == npan + R) {
        if (mine > 0)
          each_flagged([&](int pos, int col) {
            idx[pos] = col;
            if (user_idx) user_idx[pos] = col;
          });
        if (tid == 0) {
          *cnt = total;
          if (user_cnt) *user_cnt = total;
        }
        return;
      }
      // panel workgroups: the first kPanelCols outlier columns, then one
      // value of a panel per thread (zeros past the outlier count)
      __shared__ int pcol[kPanelCols];
      if (mine > 0 && before < kPanelCols)
        each_flagged([&](int pos, int col) {
          if (pos < kPanelCols) pcol[pos] = col;
        });
      __syncthreads();
      const int np = total < kPanelCols ? total : kPanelCols;
      const int j = tid % kPanelCols;
      const int cj = j < np ? pcol[j] : 0;
      if (bid < nxp) {
        const int64_t r = bid * kPanelRows + tid / kPanelCols;
        if (r < R) {
          const uint16_t v = ((const uint16_t*)x)[r * K + cj];
          pan.x_panel[r * kPanelCols + j] = j < np ? v : (uint16_t)0;
        }
      } else {
        const int64_t n = (bid - nxp) * kPanelRows + tid / kPanelCols;
        if (n < pan.N) {
          const float s = pan.w_scale[n], z = (float)(int)pan.w_zp[n];
          const uint16_t v = __builtin_bit_cast(uint16_t, outlier_weight_f16(s, pan.wq[n * K + cj], z));
          pan.w_panel[n * kPanelCols + j] = j < np ? v : (uint16_t)0;
        }
      }
      return;
    }
    bid -= npan;
  }

  const int64_t m = bid;
  const int nch = (int)(K / E);
  const int64_t row = m * K;
  const bool masked = MODE == RM_I8_OUTLIER && flags != nullptr;
  auto flag_word = [&](int c) -> uint64_t {
    if constexpr (MODE == RM_I8_OUTLIER) return masked ? *(const uint64_t*)(flags + (int64_t)c * 8) : 0;
    return 0;
  };
  auto values = [&](const v4i& ch, uint64_t f, float* v) {
    Chunk<DT>::decode(ch, v);
    if constexpr (MODE == RM_I8_OUTLIER) {
      if (__any(f != 0)) {
#pragma unroll
        for (int e = 0; e < E; ++e)
          if ((f >> (8 * e)) & 0xffu) v[e] = 0.0f;
      }
    }
  };

  v4i d[CACHE];
  uint64_t fw[CACHE];
#pragma unroll
  for (int j = 0; j < CACHE; ++j) {
    const int c = tid + kThreads * j;
    if (c < nch) {
      d[j] = load_chunk<DT>(x, row, c);
      fw[j] = flag_word(c);
    }
  }
  float amax = 0.0f;
  auto take_max = [&](const v4i& ch, uint64_t f) {
    float v[E];
    values(ch, f, v);
#pragma unroll
    for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(v[e]));
  };
  if constexpr (MODE != RM_I8_STATIC) {
#pragma unroll
    for (int j = 0; j < CACHE; ++j)
      if (tid + kThreads * j < nch) take_max(d[j], fw[j]);
    for (int c = tid + kThreads * CACHE; c < nch; c += kThreads) take_max(load_chunk<DT>(x, row, c), flag_word(c));
    amax = block_max<kWaves>(amax, redf);
  }

  float s;
  bool fast;   // the two-FMA quotient applies where the scale comes from a 16-bit row absmax
  if constexpr (MODE == RM_FP8) {
    const float a = fminf(amax, bound);
    s = a / kFp8Max;
    fast = (DT != DT_F32) && (amax <= bound);
  } else if constexpr (MODE == RM_I8_STATIC) {
    s = bound;           // the calibrated scale, used as given (no floor)
    fast = false;        // the two-FMA quotient needs a scale taken from the row absmax
  } else {
    s = amax / 127.0f;
    fast = DT != DT_F32;
  }
  if constexpr (MODE != RM_I8_STATIC) s = s < kEps ? kEps : s;
  const float r = 1.0f / s;
  // the product path of a static scale needs r to carry its full precision
  const bool r_normal = __builtin_isnormal(r);
  int qsum = 0;
  auto emit = [&](const v4i& ch, uint64_t f, int c) {
    float v[E];
    values(ch, f, v);
    uint32_t words[E / 4];
#pragma unroll
    for (int g = 0; g < E / 4; ++g) {
      if constexpr (MODE == RM_FP8) {
        float q[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float xv = v[4 * g + e];
          const float y = fast ? __builtin_copysignf(quot_fma(xv, s, r), xv) : xv / s;
          q[e] = fminf(fmaxf(y, -kFp8Max), kFp8Max);
        }
        words[g] = pack4_e4m3(q[0], q[1], q[2], q[3]);
      } else {
        // |x / s| <= 127 (s = absmax/127 rounded, or the 1e-8 floor), so the
        // codes need no clamp and the 1.5 * 2^23 rounding applies; a static
        // scale needs the clamp (clamping before rounding to even is the same
        // for the integer bounds +-127)
        uint32_t b[4];
        if constexpr (MODE == RM_I8_STATIC) {
          // A static scale: the code of RN(x / s) from one product t = RN(x r),
          // r = RN(1 / s).  |t - x/s| <= 2^-23 |x/s| (< 2^-16 below 128) and
          // RN(x/s) is within half an ulp (<= 2^-18) of x/s, so where t lies
          // more than 2^-14 from every half-integer both round to the same
          // integer, and the clamp to +-127 keeps them equal; from |t| >= 128
          // on, |x/s| > 127.5 too and both saturate (t = +-inf gives a NaN
          // distance, hence no tie).  The few values next to a half-integer
          // (and every value when r is not a normal number) take the division
          // itself.
          float y[4];
          bool near[4];
          bool any_near = false;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float t = v[4 * g + e] * r;
            const float d = fabsf(t - __builtin_rintf(t)) - 0.5f;
            near[e] = !r_normal || fabsf(d) <= 0x1p-14f;
            any_near |= near[e];
            y[e] = fminf(fmaxf(t, -127.0f), 127.0f);
          }
          if (__any(any_near)) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (near[e]) y[e] = fminf(fmaxf(v[4 * g + e] / s, -127.0f), 127.0f);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) b[e] = rne_int8_bits(y[e]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float xv = v[4 * g + e];
            b[e] = rne_int8_bits(fast ? quot_fma(xv, s, r) : xv / s);
          }
        }
        words[g] = pack_lo_bytes(b[0], b[1], b[2], b[3]);
        qsum = sum_i8x4(words[g], qsum);
      }
    }
    store_codes<E>(xq, row + (int64_t)c * E, words);
    if constexpr (MODE == RM_I8_GROUPS) {
      // chunk c belongs to group c / glanes; its glanes chunks (8, 16 or 32:
      // groups of 64 or 128 values) sit in glanes consecutive lanes of one
      // wave (chunk c is thread c % 256), all active together since K is a
      // multiple of the group size.  The sum runs on DPP moves inside the
      // 16-lane rows (quad swaps, then the half-row and row mirrors); one
      // lane permute joins two rows for 32 lanes.
      int cs = 0;
#pragma unroll
      for (int g = 0; g < E / 4; ++g) cs = sum_i8x4(words[g], cs);
      cs += __builtin_amdgcn_update_dpp(0, cs, 0xB1, 0xF, 0xF, false);
      cs += __builtin_amdgcn_update_dpp(0, cs, 0x4E, 0xF, 0xF, false);
      cs += __builtin_amdgcn_update_dpp(0, cs, 0x141, 0xF, 0xF, false);
      if (glanes >= 16) cs += __builtin_amdgcn_update_dpp(0, cs, 0x140, 0xF, 0xF, false);
      if (glanes >= 32) cs += __shfl_xor(cs, 16, 64);
      if ((c & (glanes - 1)) == 0) gsum[(int64_t)(c / glanes) * R + m] = cs;
    }
  };
#pragma unroll
  for (int j = 0; j < CACHE; ++j) {
    const int c = tid + kThreads * j;
    if (c < nch) emit(d[j], fw[j], c);
  }
  for (int c = tid + kThreads * CACHE; c < nch; c += kThreads) emit(load_chunk<DT>(x, row, c), flag_word(c), c);
  if constexpr (MODE != RM_FP8) qsum = block_sum<kWaves>(qsum, redi);
  if (tid == 0) {
    if (x_scale) x_scale[m] = s;
    if (MODE != RM_FP8 && x_rowsum) x_rowsum[m] = qsum;
  }
}

template <int MODE>
void launch_rows(const void* x, int dt, int64_t R, int64_t K, const uint8_t* flags, float bound, uint8_t* xq,
                 float* x_scale, int32_t* x_rowsum, int32_t* idx, int32_t* cnt, int32_t* user_idx,
                 int32_t* user_cnt, unsigned grid, hipStream_t st, int32_t* gsum = nullptr, int glanes = 0) {
  const OutlierPanels none{};
  const bool small = K <= 8 * kSmallCache * kThreads;   // 16-bit rows: at most kSmallCache chunks per thread
  switch (dt) {
    case DT_F32:
      k_quant_rows<MODE, DT_F32><<<grid, kThreads, 0, st>>>(x, R, K, flags, bound, xq, x_scale, x_rowsum, idx,
                                                            cnt, user_idx, user_cnt, gsum, glanes, none);
      break;
    case DT_F16:
      if (small)
        k_quant_rows<MODE, DT_F16, kSmallCache><<<grid, kThreads, 0, st>>>(
            x, R, K, flags, bound, xq, x_scale, x_rowsum, idx, cnt, user_idx, user_cnt, gsum, glanes, none);
      else
        k_quant_rows<MODE, DT_F16><<<grid, kThreads, 0, st>>>(x, R, K, flags, bound, xq, x_scale, x_rowsum, idx,
                                                              cnt, user_idx, user_cnt, gsum, glanes, none);
      break;
    default:
      if (small)
        k_quant_rows<MODE, DT_BF16, kSmallCache><<<grid, kThreads, 0, st>>>(
            x, R, K, flags, bound, xq, x_scale, x_rowsum, idx, cnt, user_idx, user_cnt, gsum, glanes, none);
      else
        k_quant_rows<MODE, DT_BF16><<<grid, kThreads, 0, st>>>(x, R, K, flags, bound, xq, x_scale, x_rowsum, idx,
                                                               cnt, user_idx, user_cnt, gsum, glanes, none);
      break;
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
  launch_rows<RM_FP8>(x, dt, R, K, nullptr, bound, xq, x_scale, nullptr, nullptr, nullptr, nullptr, nullptr,
                      (unsigned)R, st);
  return hipGetLastError();
}

hipError_t launch_quant_act_i8(const void* x, int dt, int64_t M, int64_t K, int8_t* xq, float* x_scale,
                               int32_t* x_rowsum, hipStream_t st) {
  launch_rows<RM_I8>(x, dt, M, K, nullptr, 0.0f, (uint8_t*)xq, x_scale, x_rowsum, nullptr, nullptr, nullptr,
                     nullptr, (unsigned)M, st);
  return hipGetLastError();
}

hipError_t launch_quant_act_i8_static(const void* x, int dt, int64_t M, int64_t K, float scale, int8_t* xq,
                                      float* x_scale, int32_t* x_rowsum, hipStream_t st) {
  launch_rows<RM_I8_STATIC>(x, dt, M, K, nullptr, scale, (uint8_t*)xq, x_scale, x_rowsum, nullptr, nullptr, nullptr,
                            nullptr, (unsigned)M, st);
  return hipGetLastError();
}

hipError_t launch_quant_act_i8_groups(const void* x, int dt, int64_t M, int64_t K, int64_t group, int8_t* xq,
                                      float* x_scale, int32_t* gsum, hipStream_t st) {
  const int elems = dt == DT_F32 ? 4 : 8;   // values per 16-byte chunk
  launch_rows<RM_I8_GROUPS>(x, dt, M, K, nullptr, 0.0f, (uint8_t*)xq, x_scale, nullptr, nullptr, nullptr, nullptr,
                            nullptr, (unsigned)M, st, gsum, (int)(group / elems));
  return hipGetLastError();
}

hipError_t launch_quant_act_f16_outliers(const uint16_t* x, int64_t M, int64_t K, const uint8_t* flags,
                                         int8_t* xq, float* x_scale, int32_t* x_rowsum, int32_t* idx,
                                         int32_t* cnt, int32_t* user_idx, int32_t* user_cnt,
                                         const OutlierPanels& p, hipStream_t st) {
  // the panel workgroups (16 rows each), one workgroup per row, then the
  // compaction workgroup
  constexpr int kPanelRows = kThreads / kPanelCols;
  const int64_t panels =
      p.x_panel != nullptr ? (M + kPanelRows - 1) / kPanelRows + (p.N + kPanelRows - 1) / kPanelRows : 0;
  if (K <= 8 * kSmallCache * kThreads)
    k_quant_rows<RM_I8_OUTLIER, DT_F16, kSmallCache><<<(unsigned)(M + 1 + panels), kThreads, 0, st>>>(
        x, M, K, flags, 0.0f, (uint8_t*)xq, x_scale, x_rowsum, idx, cnt, user_idx, user_cnt, nullptr, 0, p);
  else
    k_quant_rows<RM_I8_OUTLIER, DT_F16><<<(unsigned)(M + 1 + panels), kThreads, 0, st>>>(
        x, M, K, flags, 0.0f, (uint8_t*)xq, x_scale, x_rowsum, idx, cnt, user_idx, user_cnt, nullptr, 0, p);
  return hipGetLastError();
}

}  // namespace q8
