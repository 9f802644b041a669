// Weight-only W8A16 linear for decode-sized M (<= 16 tokens): the int8
// asymmetric weights are widened in registers and multiplied with the 16-bit
// activations as they are ("lecture notes on LLM quantization", PTQ section,
// weight quantization: INT8 weights read from memory and dequantized for a
// 16-bit product; no activation quantization):
//     y[m,n] = S_w[n] Sum_k x[m,k] (q[n,k] - Z_w[n])  (+ b[n])
//
// The layout is the decode kernel's: a workgroup owns 16 weight rows and its
// 4 waves split each 4096-wide K segment into 1024-column shares; each wave
// copies its share of the M activation rows into its own LDS region (DMA) and
// streams its 16 weight loads of 16 bytes (non-temporal buffer loads), then
// runs v_mfma_f32_16x16x32_{bf16,f16} with the widened weights as A (rows n)
// and the activations as B (columns m).  Each 16-byte weight chunk feeds two
// MFMAs (bytes 0-7 and 8-15); the activations follow the same k order.
//
// Widening, exact in both formats:
//   bf16  the byte is offset to u = q + 128 in [0, 255] (one xor per 4
//         bytes), converted with v_cvt_f32_ubyte and packed to bf16 (8
//         significant bits hold any u exactly).  The offset comes back through
//         sum_k x: a second MFMA with an all-ones A gives it in the same
//         output layout, and y = S_w (acc - (Z_w + 128) sum_k x).
//   f16   the bytes are placed under the exponent byte 0x64 (v_perm: f16
//         value 1024 + u), and one packed f16 add of -(1024 + 128 + Z_w) gives
//         q - Z_w exactly (|q - Z_w| <= 255 < 2^11); y = S_w acc.
// The products are exact in the fp32 accumulator; only the accumulation
// order rounds.
//
// Weight columns past K read the next row's bytes (or, past the matrix, the
// zeros of the buffer range check); the activation chunks there are zeroed,
// so they add nothing.  Activation rows m >= M repeat row M-1 and only feed
// output columns that are not stored.
#include "q8_device.hpp"
#include "q8_kernels.hpp"

namespace q8 {
namespace {

constexpr int kRows = 16;                // weight rows per workgroup
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kSeg = 4096;               // K columns per segment
constexpr int kKW = kSeg / kWaves;       // columns of a segment per wave
constexpr int kSteps = kKW / 64;         // 16-byte weight chunks per lane per segment
constexpr int kXPitch = 2 * kKW + 16;    // LDS bytes per activation row of a wave's share

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Two 8-value halves of one 16-byte weight chunk, widened to 16-bit A operands.
template <int DT>
__device__ __forceinline__ void widen(const v4i w, uint32_t zfix, v4i& lo, v4i& hi) {
  int out[8];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t u = (uint32_t)w[d] ^ 0x80808080u;   // q + 128 in each byte
    if constexpr (DT == DT_BF16) {
      const float f0 = (float)(u & 0xff), f1 = (float)((u >> 8) & 0xff);
      const float f2 = (float)((u >> 16) & 0xff), f3 = (float)(u >> 24);
      // bf16 = the high half of the exact fp32 value
      out[2 * d] = (int)__builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
      out[2 * d + 1] = (int)__builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
    } else {
      // f16 halves 0x64uu = 1024 + u, then + (-(1152 + Z)) packed: q - Z
      const uint32_t p01 = __builtin_amdgcn_perm(0x64646464u, u, 0x05010400u);
      const uint32_t p23 = __builtin_amdgcn_perm(0x64646464u, u, 0x07030602u);
      typedef _Float16 h2 __attribute__((ext_vector_type(2)));
      const h2 z = __builtin_bit_cast(h2, zfix);
      out[2 * d] = __builtin_bit_cast(int, __builtin_bit_cast(h2, p01) + z);
      out[2 * d + 1] = __builtin_bit_cast(int, __builtin_bit_cast(h2, p23) + z);
    }
  }
  lo = v4i{out[0], out[1], out[2], out[3]};
  hi = v4i{out[4], out[5], out[6], out[7]};
}

template <int DT>
__device__ __forceinline__ v4f mma16(const v4i a, const v4i b, const v4f c) {
  if constexpr (DT == DT_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0,
                                                   0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
}

template <int DT, int YDT>
__global__ __launch_bounds__(kThreads, 1) void k_gemv_w8a16(const uint16_t* __restrict__ x, int M, int K,
                                                            const int8_t* __restrict__ wq,
                                                            const float* __restrict__ w_scale,
                                                            const float* __restrict__ w_zp, int N,
                                                            const float* __restrict__ bias, void* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint8_t xs[kWaves][kRows * kXPitch];
  __shared__ v4f part[kWaves][64];
  __shared__ v4f psum[kWaves][64];
  // per-channel factors of the 16 columns, one 1 KB DMA by wave 0: scales at
  // [0, 16), zero points at [16, 32), biases at [32, 48)
  __shared__ __attribute__((aligned(16))) float fac[256];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * kRows;
  uint8_t* const xw = xs[wave];
  const int wrow = n0 + lr < N ? n0 + lr : N - 1;
  const __amdgpu_buffer_rsrc_t wres = byte_buffer(wq, (uint32_t)N * (uint32_t)K);
  // f16: the packed addend -(1024 + 128 + Z) of this lane's row, twice; the
  // zero point is loaded now and used only after the activations' wait
  float zraw = DT == DT_F16 ? w_zp[wrow] : 0.0f;
  uint32_t zfix = 0;
  const int xr = lr < M ? lr : M - 1;
  const v4i ones = DT == DT_BF16 ? v4i{0x3f803f80, 0x3f803f80, 0x3f803f80, 0x3f803f80} : v4i{0, 0, 0, 0};
  v4f acc = {0.0f, 0.0f, 0.0f, 0.0f}, accs = {0.0f, 0.0f, 0.0f, 0.0f};
  // Epilogue factors (wave 0).  With all 16 columns present they come by one
  // DMA between the two halves of the first segment's weight loads: they
  // neither delay the activations nor arrive after the last weight.
  // Otherwise (the last workgroup of a ragged N) by vector loads here, ahead
  // of the activations.  (Vector loads after the weights, by wave 0 only,
  // made the compiler's merged wait count hold wave 0's first MFMA until
  // nearly all its weights had arrived.)
  const bool fac_dma = n0 + kRows <= N;
  float fsc[4] = {0, 0, 0, 0}, fzp[4] = {0, 0, 0, 0}, fbi[4] = {0, 0, 0, 0};
  if (wave == 0 && !fac_dma) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = n0 + 4 * lg + r;
      const int nc = n < N ? n : N - 1;
      fsc[r] = w_scale[nc];
      fzp[r] = w_zp[nc];
      fbi[r] = bias ? bias[nc] : 0.0f;
    }
  }

  for (int k0 = 0; k0 < K; k0 += kSeg) {
    const int seg = (K - k0) < kSeg ? (K - k0) : kSeg;
    if (k0 > 0) __builtin_amdgcn_s_waitcnt(kLgkmcnt0);   // this wave's reads of the last segment are done
    // the wave's share of each activation row: two 1 KB DMAs (512 values each)
    for (int m = 0; m < M; ++m) {
      const uint8_t* base = (const uint8_t*)x + ((size_t)m * K + k0) * 2;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        int c = wave * kKW + 512 * j + 8 * lane;
        c = c < seg ? c : seg - 8;                      // clamped: zeroed after the read
        dma16(base, (uint32_t)c * 2, xw + m * kXPitch + 1024 * j);
      }
    }
    v4i wv[kSteps];
    const uint32_t wbase = (uint32_t)(wrow * K + k0 + wave * kKW + lg * 16);
    const bool fdma = k0 == 0 && fac_dma && wave == 0;
#pragma unroll
    for (int s = 0; s < kSteps / 2; ++s) wv[s] = load16_nt(wres, wbase + s * 64);
    if (fdma) {
      // lane l: chunk l % 4 of the scales (l < 4 or l >= 12), zero points
      // (4 <= l < 8) or biases (8 <= l < 12)
      const int arr = lane >> 2;
      const float* src = arr == 1 ? w_zp : (arr == 2 && bias ? bias : w_scale);
      dma16_ptr(src + n0 + 4 * (lane & 3), (uint8_t*)fac);
    }
#pragma unroll
    for (int s = kSteps / 2; s < kSteps; ++s) wv[s] = load16_nt(wres, wbase + s * 64);
    // the activations are in: everything but the 16 weight loads issued last
    // (and the factor DMA among them)
    if (fdma) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kSteps + 1) : "memory");
    else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kSteps) : "memory");
    if constexpr (DT == DT_F16) {
      if (k0 == 0) {
        asm volatile("" : "+v"(zraw));
        const _Float16 h = (_Float16)(-(1152.0f + zraw));
        const uint32_t hb = (uint32_t)__builtin_bit_cast(uint16_t, h);
        zfix = hb | (hb << 16);
      }
    }
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      v4i a0, a1;
      widen<DT>(wv[s], zfix, a0, a1);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = wave * kKW + s * 64 + lg * 16 + 8 * j;   // first of the lane's 8 columns
        v4i b = *(const v4i*)(xw + xr * kXPitch + (c - wave * kKW) * 2);
        if (seg != kSeg && c >= seg) b = v4i{0, 0, 0, 0};
        acc = mma16<DT>(j == 0 ? a0 : a1, b, acc);
        if constexpr (DT == DT_BF16) accs = mma16<DT>(ones, b, accs);
      }
      // one k-step at a time, in order: left free, the scheduler hoists the
      // widening of many k-steps above the first MFMAs, and with it the
      // waits for their weights
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  part[wave][lane] = acc;
  psum[wave][lane] = accs;
  __syncthreads();
  if (wave == 0 && fac_dma) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the factor DMA (this wave's)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      fsc[r] = fac[4 * lg + r];
      fzp[r] = fac[16 + 4 * lg + r];
      fbi[r] = bias ? fac[32 + 4 * lg + r] : 0.0f;
    }
  }
  if (wave == 0 && lr < M) {
    v4f t = part[0][lane], ts = psum[0][lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      t += part[w][lane];
      ts += psum[w][lane];
    }
    // the factors are first used here; the empty asm keeps their conversion
    // from being hoisted next to the loads
#pragma unroll
    for (int r = 0; r < 4; ++r) asm volatile("" : "+v"(fsc[r]), "+v"(fzp[r]), "+v"(fbi[r]));
    const int m = lr;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = n0 + 4 * lg + r;
      if (n < N) {
        // register r of lane (lr, lg) is D[n = 4 lg + r][m = lr]
        const float a = DT == DT_BF16 ? t[r] - (fzp[r] + 128.0f) * ts[r] : t[r];
        float v = fsc[r] * a;
        if (bias) v += fbi[r];
        store_out<YDT>(y, (size_t)m * N + n, v);
      }
    }
  }
}

template <int DT>
hipError_t launch_dt(const uint16_t* x, int64_t M, int64_t K, const int8_t* wq, const float* ws, const float* wz,
                     int64_t N, const float* bias, void* y, int ydt, hipStream_t st) {
  dim3 grid((unsigned)((N + kRows - 1) / kRows)), block(kThreads);
  const int m = (int)M, k = (int)K, n = (int)N;
  switch (ydt) {
    case DT_F32: k_gemv_w8a16<DT, DT_F32><<<grid, block, 0, st>>>(x, m, k, wq, ws, wz, n, bias, y); break;
    case DT_F16: k_gemv_w8a16<DT, DT_F16><<<grid, block, 0, st>>>(x, m, k, wq, ws, wz, n, bias, y); break;
    default: k_gemv_w8a16<DT, DT_BF16><<<grid, block, 0, st>>>(x, m, k, wq, ws, wz, n, bias, y); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_w8a16(const void* x, int xdt, int64_t M, int64_t K, const int8_t* wq, const float* w_scale,
                             const float* w_zp, int64_t N, const float* bias, void* y, int ydt, hipStream_t st) {
  const uint16_t* xx = static_cast<const uint16_t*>(x);
  if (xdt == DT_F16) return launch_dt<DT_F16>(xx, M, K, wq, w_scale, w_zp, N, bias, y, ydt, st);
  return launch_dt<DT_BF16>(xx, M, K, wq, w_scale, w_zp, N, bias, y, ydt, st);
}

}  // namespace q8
