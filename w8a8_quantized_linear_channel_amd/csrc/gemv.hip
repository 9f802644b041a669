// Decode-shaped W8A8 linear (M <= 16 tokens): one launch that quantizes the
// activations per token and streams the int8 weights at HBM rate.
//
// A workgroup owns 16 weight rows (output features) and all of K; the grid is
// ceil(N / 16) workgroups (256 for the 4096-row q_proj, one per CU).  Its 8
// waves split into two roles so the two latencies overlap:
//   * 4 "streamer" waves issue every 16-byte load of their weight rows for
//     the current K segment up front (64 KB in flight per workgroup at
//     K = 4096), then run v_mfma_i32_16x16x64_i8 with the weights as the
//     A operand (rows n) and the activation codes from LDS as B (columns m);
//   * 4 "quantizer" waves meanwhile read X (L2-resident: at most 16 rows),
//     take each row's absmax, and write the int8 codes of the segment to LDS
//     together with the per-row code sum.
// Loads of one wave retire in order, so giving the weight stream and the
// activation reads to different waves is what lets them overlap; the weight
// loads are unconditional (clamped addresses) so nothing makes a streamer wait
// for them before the MFMAs.  Code positions past K and rows past M are zero
// in LDS, so whatever the clamped weight loads bring there adds nothing.
// The four streamers' partial INT32 tiles are summed through LDS and one wave
// applies the epilogue y = S_x S_w (acc - Z_w sum_k q_x) (+ bias).
#include "q8_device.hpp"
#include "q8_kernels.hpp"

namespace q8 {
namespace {

constexpr int kRows = 16;               // weight rows per workgroup
constexpr int kSeg = 4096;              // K bytes per LDS segment
constexpr int kStreamers = 4, kQuantizers = 4;
constexpr int kThreads = 64 * (kStreamers + kQuantizers);
constexpr int kStepsPerWave = kSeg / 64 / kStreamers;   // 16 x 16-byte loads per lane
constexpr int kXStride = kSeg + 16;     // padded LDS row: 8 rows of one column hit 8 bank groups

template <int DT, int YDT>
__global__ __launch_bounds__(kThreads, 1) void k_gemv_i8(const void* __restrict__ x, int M, int64_t K,
                                                         const int8_t* __restrict__ wq,
                                                         const float* __restrict__ w_scale,
                                                         const float* __restrict__ w_zp, int64_t N,
                                                         const float* __restrict__ bias, void* __restrict__ y,
                                                         int32_t* __restrict__ acc_out) {
  constexpr int E = Chunk<DT>::kElems;
  constexpr int esz = (DT == DT_F32) ? 4 : 2;
  constexpr int CPL = kSeg / E / 64;    // chunks per lane for one row-segment
  __shared__ __attribute__((aligned(16))) int8_t xs[kRows * kXStride];
  __shared__ float sx[kRows];
  __shared__ int rsum[kRows];
  __shared__ v4i part[kStreamers][64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * kRows;
  const char* xb = (const char*)x;

  // ---- streamers: every weight load of a K segment in flight at once
  v4i wv[kStepsPerWave];
  const int64_t wrow = (n0 + lr < N ? n0 + lr : N - 1) * K;
  auto issue = [&](int64_t k0) {
    const int seg = (int)((K - k0) < kSeg ? (K - k0) : kSeg);
#pragma unroll
    for (int j = 0; j < kStepsPerWave; ++j) {
      int kk = (wave + j * kStreamers) * 64 + lg * 16;
      kk = kk < seg ? kk : seg - 16;
      wv[j] = *(const v4i*)(wq + wrow + k0 + kk);
    }
  };

  // ---- quantizers: one row-segment of X is CPL chunks per lane
  auto load_seg = [&](int m, int64_t k0, int seg, v4i* ch) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + 64 * j;
      ch[j] = c < seg / E ? *(const v4i*)(xb + ((int64_t)m * K + k0 + (int64_t)c * E) * esz)
                          : v4i{0, 0, 0, 0};
    }
  };
  auto seg_absmax = [&](const v4i* ch) {
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      float v[E];
      Chunk<DT>::decode(ch[j], v);
#pragma unroll
      for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(v[e]));
    }
    return amax;
  };
  // codes of one row-segment into LDS; returns this lane's code sum.  For
  // 16-bit inputs the quotient comes from two FMAs on RN(1/s) (same codes as
  // the division for a scale taken from the row absmax).
  auto seg_codes = [&](int m, int seg, const v4i* ch, float s, float r) {
    int qsum = 0;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + 64 * j;
      if (c < seg / E) {
        float v[E];
        Chunk<DT>::decode(ch[j], v);
        uint32_t words[E / 4];
#pragma unroll
        for (int gq = 0; gq < E / 4; ++gq) {
          uint32_t b[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float xv = v[4 * gq + e];
            b[e] = rne_int8_bits(DT == DT_F32 ? xv / s : quot_fma(xv, s, r));
          }
          words[gq] = pack_lo_bytes(b[0], b[1], b[2], b[3]);
          qsum = sum_i8x4(words[gq], qsum);
        }
        if constexpr (E == 8) {
          *(v2i*)(xs + m * kXStride + c * E) = v2i{(int)words[0], (int)words[1]};
        } else {
          *(uint32_t*)(xs + m * kXStride + c * E) = words[0];
        }
      }
    }
    return qsum;
  };

  const int qw = wave - kStreamers;
  const bool one_seg = K <= kSeg;
  v4i cur[CPL];
  if (wave < kStreamers) {
    issue(0);
  } else {
    // rows M..15 of the code buffer stay zero for every segment
    for (int i = qw * 64 + lane; i < (kRows - M) * (kSeg / 16); i += kQuantizers * 64) {
      const int m = M + i / (kSeg / 16), c = i % (kSeg / 16);
      *(v4i*)(xs + m * kXStride + c * 16) = v4i{0, 0, 0, 0};
    }
    if (!one_seg) {
      // per-row absmax over every segment of the row
      for (int m = qw; m < M; m += kQuantizers) {
        float amax = 0.0f;
        for (int64_t k0 = 0; k0 < K; k0 += kSeg) {
          const int seg = (int)((K - k0) < kSeg ? (K - k0) : kSeg);
          load_seg(m, k0, seg, cur);
          amax = fmaxf(amax, seg_absmax(cur));
        }
        amax = wave_max(amax);
        float s = amax / 127.0f;
        s = s < kEps ? kEps : s;
        if (lane == 0) { sx[m] = s; rsum[m] = 0; }
      }
    }
  }

  v4i acc = {0, 0, 0, 0};
  for (int64_t k0 = 0; k0 < K; k0 += kSeg) {
    const int seg = (int)((K - k0) < kSeg ? (K - k0) : kSeg);
    __syncthreads();   // the previous segment's codes have been consumed
    if (wave >= kStreamers) {
      // a partial segment: code positions past K are zero
      if (seg < kSeg) {
        for (int m = qw; m < M; m += kQuantizers)
          for (int b = seg + lane * 16; b < kSeg; b += 64 * 16) *(v4i*)(xs + m * kXStride + b) = v4i{0, 0, 0, 0};
      }
      // rows of this wave, the next row's loads in flight while one is coded
      v4i nxt[CPL];
      if (qw < M) load_seg(qw, k0, seg, cur);
      for (int m = qw; m < M; m += kQuantizers) {
        if (m + kQuantizers < M) load_seg(m + kQuantizers, k0, seg, nxt);
        float s;
        if (one_seg) {
          const float amax = wave_max(seg_absmax(cur));
          s = amax / 127.0f;
          s = s < kEps ? kEps : s;
        } else {
          s = sx[m];
        }
        const float r = 1.0f / s;
        const int qsum = wave_sum(seg_codes(m, seg, cur, s, r));
        if (lane == 0) {
          if (one_seg) { sx[m] = s; rsum[m] = qsum; }
          else rsum[m] += qsum;
        }
#pragma unroll
        for (int j = 0; j < CPL; ++j) cur[j] = nxt[j];
      }
    }
    __syncthreads();   // the codes of this segment are in LDS
    if (wave < kStreamers) {
#pragma unroll
      for (int j = 0; j < kStepsPerWave; ++j) {
        const int st = wave + j * kStreamers;
        const v4i xv = *(const v4i*)(xs + lr * kXStride + st * 64 + lg * 16);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wv[j], xv, acc, 0, 0, 0);
      }
      if (k0 + kSeg < K) issue(k0 + kSeg);
    }
  }

  // ---- sum the streamers' partial tiles, epilogue.  acc register r of lane
  // (lr, lg) is D[n = 4*lg + r][m = lr].
  if (wave < kStreamers) part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    v4i t = part[0][lane];
#pragma unroll
    for (int w = 1; w < kStreamers; ++w) t += part[w][lane];
    const int m = lr;
    if (m < M) {
      const float s_m = sx[m];
      const int r_m = rsum[m];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t n = n0 + lg * 4 + r;
        if (n < N) {
          const int a = t[r];
          if (acc_out) acc_out[(int64_t)m * N + n] = a;
          const int c = a - (int)w_zp[n] * r_m;
          float v = (s_m * w_scale[n]) * (float)c;
          if (bias) v += bias[n];
          store_out<YDT>(y, (int64_t)m * N + n, v);
        }
      }
    }
  }
}

template <int DT>
hipError_t launch_dt(const void* x, int64_t M, int64_t K, const int8_t* wq, const float* ws,
                     const float* wz, int64_t N, const float* bias, void* y, int ydt, int32_t* acc_out,
                     hipStream_t st) {
  dim3 grid((unsigned)((N + kRows - 1) / kRows)), block(kThreads);
  switch (ydt) {
    case DT_F32: k_gemv_i8<DT, DT_F32><<<grid, block, 0, st>>>(x, (int)M, K, wq, ws, wz, N, bias, y, acc_out); break;
    case DT_F16: k_gemv_i8<DT, DT_F16><<<grid, block, 0, st>>>(x, (int)M, K, wq, ws, wz, N, bias, y, acc_out); break;
    default: k_gemv_i8<DT, DT_BF16><<<grid, block, 0, st>>>(x, (int)M, K, wq, ws, wz, N, bias, y, acc_out); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_i8(const void* x, int xdt, int64_t M, int64_t K, const int8_t* wq,
                          const float* w_scale, const float* w_zp, int64_t N, const float* bias,
                          void* y, int ydt, int32_t* acc_out, hipStream_t st) {
  switch (xdt) {
    case DT_F32: return launch_dt<DT_F32>(x, M, K, wq, w_scale, w_zp, N, bias, y, ydt, acc_out, st);
    case DT_F16: return launch_dt<DT_F16>(x, M, K, wq, w_scale, w_zp, N, bias, y, ydt, acc_out, st);
    default: return launch_dt<DT_BF16>(x, M, K, wq, w_scale, w_zp, N, bias, y, ydt, acc_out, st);
  }
}

}  // namespace q8
