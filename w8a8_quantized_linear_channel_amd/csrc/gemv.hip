// Decode-shaped W8A8 linear.  Up to ten tokens: one launch that quantizes the
// activations per token and streams the int8 weights (k_gemv_i8, below).
// From eleven to sixteen tokens the rows are quantized once by the row
// quantizer and k_gemv_q8 (further down) streams weights against the codes.
//
// A workgroup owns 16 weight rows (output features) and all of K; the grid is
// ceil(N / 16) workgroups (256 for the 4096-row q_proj, one per CU).  Its 4
// waves split K: inside each 4096-wide K segment, wave w owns the 1024
// columns [1024 w, 1024 w + 1024) for everything it does --
//   * it first copies those columns of every X row into its own LDS region
//     (global_load_lds, so no registers are held), then issues its 16
//     16-byte weight loads (16 rows x 1024 bytes, non-temporal buffer
//     loads): the activations, which every workgroup reads, are not queued
//     behind 64 KB of weight traffic;
//   * it takes each row's partial absmax over its columns; one barrier
//     combines the four partials into the row scale;
//   * it overwrites each row's X values in LDS with their int8 codes and runs
//     v_mfma_i32_16x16x64_i8 over them with the weights as the A operand
//     (rows n) and the codes as B (columns m).  Only this wave touches the
//     region, so no barrier is needed between coding and the MFMAs.
// Rows are processed in run-time loops: the kernel runs once per call, so
// every instruction is fetched cold, and compact code is what keeps the
// activation work short.  Each k-step also runs an MFMA of all-ones weights
// against the codes, which gives sum_k q_x in the accumulator's own layout;
// the four partial INT32 tiles and code sums meet in LDS and wave 0 applies
// y = S_x S_w (acc - Z_w sum_k q_x) (+ bias) with the per-row factors it
// loaded at the start.
//
// Code columns past K are zero, so the clamped weight loads there add
// nothing.  Code rows m >= M hold stale bytes: they only feed MFMA output
// columns that are not stored.
#include "q8_device.hpp"
#include "q8_group.hpp"
#include "q8_kernels.hpp"

namespace q8 {
namespace {

constexpr int kRows = 16;               // weight rows per workgroup
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kSeg = 4096;              // K columns per segment
constexpr int kKW = kSeg / kWaves;      // columns of a segment per wave (1024)
constexpr int kSteps = kKW / 64;        // 64-byte MFMA k-steps per wave per segment (16)
// One row's area in a wave's LDS region: 1024 16-bit X values (2048 bytes),
// later overwritten by their 1024 codes.  The 16-byte pad puts the 16 code
// rows read by one MFMA operand fetch in 16 different bank quarters.
constexpr int kArea = 2 * kKW + 16;


// ONE: K <= 4096, a single segment (the host picks the instantiation, so each
// kernel has one straight path and the compiler's wait insertion sees it alone).
// GS > 0: per-group weights (groups of GS columns; w_scale / w_zp are
// group-major [K / GS, N]).  Each k-step also runs an MFMA of all-ones
// weights against the codes, which gives sum_k q_x over the step in the
// accumulator's own layout; after each group the INT32 tile is corrected by
// Z times that sum, exactly, and added into fp32 with the group's scale.
template <int DT, int YDT, bool ONE, int GS = 0>
__global__ __launch_bounds__(kThreads, 1) void k_gemv_i8(const void* __restrict__ x, int M, int K,
                                                         const int8_t* __restrict__ wq,
                                                         const float* __restrict__ w_scale,
                                                         const float* __restrict__ w_zp, int N,
                                                         const float* __restrict__ bias, void* __restrict__ y,
                                                         int32_t* __restrict__ acc_out) {
  __shared__ __attribute__((aligned(16))) uint8_t xs[kWaves][kRows * kArea];
  // Per-thread partial absmax of every row: no reduction inside the row
  // loop; one block-wide pass reduces all rows at once.
  __shared__ __attribute__((aligned(16))) float lred[kRows][kThreads];
  __shared__ float rscale[kRows];
  __shared__ v4i part[kWaves][64];
  __shared__ v4i psum[kWaves][64];     // the code sums' partial tiles
  // per-channel factors of the 16 columns, one 1 KB DMA by wave 0: scales at
  // [0, 16), zero points at [16, 32), biases at [32, 48); the rest unused
  __shared__ __attribute__((aligned(16))) float fac[256];
  // per-group weights of 128: each wave's 8 groups' scales and zero points
  // for the 16 columns, one 1 KB DMA per wave (group t's scales at
  // [32 t, 32 t + 16), its zero points at [32 t + 16, 32 t + 32))
  __shared__ __attribute__((aligned(16))) float gpar[GS == 128 ? kWaves : 1][256];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * kRows;
  const uint8_t* xb = (const uint8_t*)x;
  uint8_t* const xw = xs[wave];
  const int nseg = (K + kSeg - 1) / kSeg;
  auto seg_len = [&](int sg) __attribute__((always_inline)) { return (K - sg * kSeg) < kSeg ? (K - sg * kSeg) : kSeg; };

  // The lane's columns inside the wave's 1024: chunk j (0, 1) is columns
  // [512 j + 8 lane, 512 j + 8 lane + 8); a chunk lies wholly inside or
  // wholly outside the segment (both are multiples of 8 or 16).
  auto col = [&](int j) __attribute__((always_inline)) { return wave * kKW + 512 * j + 8 * lane; };

  // ---- X of one segment into LDS, 16-bit inputs: two 1 KB DMA per row
  auto dma_x = [&](int k0, int seg) __attribute__((always_inline)) {
    for (int m = 0; m < M; ++m) {
      const uint8_t* base = xb + ((size_t)m * K + k0) * 2;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = col(j) < seg ? col(j) : seg - 8;     // clamped: masked after the read
        dma16(base, (uint32_t)c * 2, xw + m * kArea + 1024 * j);
      }
    }
  };
  // the lane's 16 values of row m: from LDS (16-bit) or from global (fp32)
  auto get_x = [&](int m, int k0, int seg, float* v) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const bool ok = col(j) < seg;
      if constexpr (DT == DT_F32) {
        const int c = ok ? col(j) : seg - 8;
        const float* p = (const float*)xb + (size_t)m * K + k0 + c;
        const v4i a = *(const v4i*)p, b = *(const v4i*)(p + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[8 * j + e] = ok ? __int_as_float(a[e]) : 0.0f;
          v[8 * j + 4 + e] = ok ? __int_as_float(b[e]) : 0.0f;
        }
      } else {
        v4i ch = *(const v4i*)(xw + m * kArea + 1024 * j + 16 * lane);
        // a chunk past K reads as +0 (only a partial segment has one)
        if (seg != kSeg && !ok) ch = v4i{0, 0, 0, 0};
        Chunk<DT>::decode(ch, v + 8 * j);
      }
    }
  };

  // ---- weights: 16 loads of 16 bytes per lane (rows n0 + lane%16), through
  // a buffer resource over the whole matrix: one offset per lane, the 16
  // steps as immediate offsets, and the non-temporal hint, so the stream
  // does not push the activations and the code out of the caches.  Columns
  // past the segment read the next row's bytes (or, past the matrix, the
  // zeros the hardware's range check returns): their codes are zero.
  v4i wv[kSteps];
  const int wrow = (n0 + lr < N ? n0 + lr : N - 1);
  const __amdgpu_buffer_rsrc_t wres = byte_buffer(wq, (uint32_t)N * (uint32_t)K);
  auto load_w = [&](int k0) __attribute__((always_inline)) {
    const uint32_t base = (uint32_t)(wrow * K + k0 + wave * kKW + lg * 16);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) wv[s] = load16_nt(wres, base + s * 64);
  };
  // Per channel, with all 16 columns present, wave 0 requests the epilogue
  // factors by one DMA between the first and second half of its weights:
  // requested with X they delay X, and requested after the weights (as
  // vector loads, below) they arrive after the last weight and hold up the
  // epilogue.  Lane l fetches 16 bytes: chunk l % 4 of the scales (l < 4 or
  // l >= 12), zero points (4 <= l < 8) or biases (8 <= l < 12).
  // (Per group, only the biases of that DMA are used.)  With groups of 128
  // and N a multiple of 4, every wave fetches its groups' parameters the
  // same way, by one DMA after its first four weight loads: loaded after X,
  // they held the folds, and with them the MFMAs past the first group, until
  // after the last weight.  Lane l fetches 16 bytes: chunk l % 4 of the
  // scales (bit 2 of l clear) or zero points (set) of group l / 8.
  const bool fac_dma = n0 + kRows <= N;
  const bool gp_dma = GS == 128 && n0 + kRows <= N && (N & 3) == 0;
  auto load_w_first = [&]() __attribute__((always_inline)) {
    const uint32_t base = (uint32_t)(wrow * K + wave * kKW + lg * 16);
#pragma unroll
    for (int s = 0; s < kSteps / 4; ++s) wv[s] = load16_nt(wres, base + s * 64);
    if constexpr (GS == 128) {
      if (gp_dma) {
        const int G = K / GS;
        const int t = lane >> 3, g = wave * (kKW / GS) + t < G ? wave * (kKW / GS) + t : G - 1;
        const float* src = ((lane >> 2) & 1) ? w_zp : w_scale;
        dma16_ptr(src + (size_t)g * N + n0 + 4 * (lane & 3), (uint8_t*)gpar[wave]);
      }
    }
#pragma unroll
    for (int s = kSteps / 4; s < kSteps / 2; ++s) wv[s] = load16_nt(wres, base + s * 64);
    if (fac_dma && wave == 0) {
      const int arr = lane >> 2;
      const float* src = arr == 1 ? w_zp : (arr == 2 && bias ? bias : w_scale);
      dma16_ptr(src + n0 + 4 * (lane & 3), (uint8_t*)fac);
    }
#pragma unroll
    for (int s = kSteps / 2; s < kSteps; ++s) wv[s] = load16_nt(wres, base + s * 64);
  };
  // epilogue factors (wave 0): acc register r of lane (lr, lg) is
  // D[n = 4 lg + r][m = lr].
  float fsc[4] = {0, 0, 0, 0}, fzp[4] = {0, 0, 0, 0}, fbi[4] = {0, 0, 0, 0};
  auto load_factors = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = n0 + 4 * lg + r;
      const int nc = n < N ? n : N - 1;
      fsc[r] = w_scale[nc];
      fzp[r] = w_zp[nc];
      fbi[r] = bias ? bias[nc] : 0.0f;
    }
  };

  // Block-wide reduction of lred over the 256 threads, all rows at once:
  // thread t takes row t/16 and 16 of its partials, then the 16 threads of
  // the row (one DPP row) combine theirs; every one of them gets the result.
  auto reduce_rows = [&](auto op) __attribute__((always_inline)) {
    const int m = tid >> 4, sub = tid & 15;
    const v4i* src = (const v4i*)&lred[m][sub * 16];
    int r = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const v4i c = src[i];
      r = i == 0 ? op(op(c[0], c[1]), op(c[2], c[3])) : op(r, op(op(c[0], c[1]), op(c[2], c[3])));
    }
    return dpp_row_reduce(r, op);
  };
  auto fmax_bits = [](int a, int b) __attribute__((always_inline)) { return __float_as_int(fmaxf(__int_as_float(a), __int_as_float(b))); };
  auto row_scale = [&](int m) __attribute__((always_inline)) { return rscale[m]; };
  v4i acc = {0, 0, 0, 0};
  // the code sums (per-group weights: of the current group), from the
  // all-ones MFMA; and, per-group, the fp32 sum over groups
  v4i accs = {0, 0, 0, 0};
  v4f fsum = {0.0f, 0.0f, 0.0f, 0.0f};
  constexpr int NG = GS > 0 ? kKW / GS : 1;   // groups in a wave's share of a segment
  float gsc[NG][4], gzp[NG][4];
  // the parameters of this wave's groups in segment k0 (groups past K are
  // clamped and their fold is skipped)
  auto load_groups = [&](int k0) __attribute__((always_inline)) {
    if constexpr (GS > 0) {
      const int G = K / GS, g0 = (k0 + wave * kKW) / GS;
      // The lane's four columns, clamped to the last one past N (those
      // outputs are not stored), one 4-byte load each: no branch between the
      // weight loads issued before and these, since the compiler's wait
      // insertion holds loads under a branch until earlier ones (here the
      // weights) have returned.
      int nc[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) nc[r] = n0 + 4 * lg + r < N ? n0 + 4 * lg + r : N - 1;
#pragma unroll
      for (int t = 0; t < NG; ++t) {
        const int gi = g0 + t < G ? g0 + t : G - 1;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          gsc[t][r] = w_scale[gi * N + nc[r]];
          gzp[t][r] = w_zp[gi * N + nc[r]];
        }
      }
    }
  };

  // ---- pass 1 over one segment: per-row partial absmax
  auto pass1 = [&](int sg, int k0, int seg) __attribute__((always_inline)) {
    if constexpr (DT != DT_F32) {
      if (sg > 0) __builtin_amdgcn_s_waitcnt(kLgkmcnt0);   // reads of the last segment are done
      dma_x(k0, seg);
    }
    if (sg == 0) load_w_first();
    if constexpr (DT != DT_F32) {
      // this segment's X: everything but the 16 weight loads issued last
      // (and wave 0's factor DMA among them)
      if (sg > 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      else if (gp_dma && fac_dma && wave == 0) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kSteps + 2) : "memory");
      else if (gp_dma || (fac_dma && wave == 0)) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kSteps + 1) : "memory");
      else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kSteps) : "memory");
    }
    // issued after the wait, so X does not wait for them; they have the
    // whole coding and MFMA phase to arrive
    if constexpr (GS > 0) {
      if (sg == 0 && wave == 0 && !fac_dma) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = n0 + 4 * lg + r;
          fbi[r] = bias ? bias[n < N ? n : N - 1] : 0.0f;
        }
      }
      if (sg == 0 && !gp_dma) load_groups(k0);
    } else {
      if (sg == 0 && wave == 0 && !fac_dma) load_factors();
    }
#pragma unroll 4
    for (int m = 0; m < M; ++m) {
      float v[16];
      get_x(m, k0, seg, v);
      float a = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) a = fmaxf(a, fabsf(v[e]));
      lred[m][tid] = sg == 0 ? a : fmaxf(lred[m][tid], a);
    }
  };
  // row scales from the partial absmax of every thread
  auto finish_scales = [&]() __attribute__((always_inline)) {
    __syncthreads();   // every thread's partial absmax is in LDS
    const int r = reduce_rows(fmax_bits);
    if ((tid & 15) == 0 && (tid >> 4) < M) {
      const float s = __int_as_float(r) / 127.0f;
      rscale[tid >> 4] = s < kEps ? kEps : s;
    }
    __syncthreads();   // the scales are in LDS
  };
  // ---- pass 2 over one segment: codes, then the MFMAs on them.  reload:
  // X (and, past the first segment, W) must be fetched again.
  auto pass2 = [&](int sg, int k0, int seg, bool reload) __attribute__((always_inline)) {
    if (reload) {
      if constexpr (DT != DT_F32) {
        __builtin_amdgcn_s_waitcnt(kLgkmcnt0);
        dma_x(k0, seg);
      }
      if (sg > 0) load_w(k0);
      if constexpr (DT != DT_F32) {
        if (sg > 0) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kSteps) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
    }
#pragma unroll 4
    for (int m = 0; m < M; ++m) {
      float v[16];
      get_x(m, k0, seg, v);
      const float s = row_scale(m);
      const float r = 1.0f / s;
      // For 16-bit inputs the quotient comes from two FMAs on RN(1/s), which
      // gives the codes of the correctly rounded division for a scale taken
      // from the row absmax; fp32 inputs use the IEEE division.
      uint32_t words[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint32_t b[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float xv = v[4 * g + e];
          b[e] = rne_int8_bits(DT == DT_F32 ? xv / s : quot_fma(xv, s, r));
        }
        words[g] = pack_lo_bytes(b[0], b[1], b[2], b[3]);
      }
      // the row's X values have all been read (same wave, in order) before
      // their codes overwrite the start of the area
      uint8_t* area = xw + m * kArea;
      *(v2i*)(area + 8 * lane) = v2i{(int)words[0], (int)words[1]};
      *(v2i*)(area + 512 + 8 * lane) = v2i{(int)words[2], (int)words[3]};
    }
    const v4i ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
    if constexpr (GS == 0) {
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        const v4i xv = *(const v4i*)(xw + lr * kArea + s * 64 + lg * 16);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wv[s], xv, acc, 0, 0, 0);
        accs = __builtin_amdgcn_mfma_i32_16x16x64_i8(ones, xv, accs, 0, 0, 0);
      }
    } else {
      if (sg > 0) load_groups(k0);   // pass 1 loaded segment 0's groups
      if constexpr (GS == 128) {
        if (sg == 0 && gp_dma) {
          // this wave's parameter DMA: issued after its first 4 weight loads,
          // followed by 12 more (and wave 0's factor DMA)
          if (fac_dma && wave == 0) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kSteps - kSteps / 4 + 1) : "memory");
          else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kSteps - kSteps / 4) : "memory");
#pragma unroll
          for (int t = 0; t < NG; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              gsc[t][r] = gpar[wave][32 * t + 4 * lg + r];
              gzp[t][r] = gpar[wave][32 * t + 16 + 4 * lg + r];
            }
        }
      }
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        const v4i xv = *(const v4i*)(xw + lr * kArea + s * 64 + lg * 16);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wv[s], xv, acc, 0, 0, 0);
        accs = __builtin_amdgcn_mfma_i32_16x16x64_i8(ones, xv, accs, 0, 0, 0);
        if ((s + 1) % (GS / 64) == 0) {
          const int t = s / (GS / 64);
          if (wave * kKW + t * GS < seg) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int c = acc[r] - (int)gzp[t][r] * accs[r];   // exact: |c| < 2^24
              fsum[r] = fmaf(gsc[t][r], (float)c, fsum[r]);
            }
          }
          acc = v4i{0, 0, 0, 0};
          accs = v4i{0, 0, 0, 0};
        }
      }
    }
  };

  if constexpr (ONE) {
    // the common case, straight-line: X is copied once and coded in place
    pass1(0, 0, K);
    finish_scales();
    pass2(0, 0, K, false);
  } else {
    for (int sg = 0; sg < nseg; ++sg) pass1(sg, sg * kSeg, seg_len(sg));
    finish_scales();
    for (int sg = 0; sg < nseg; ++sg) pass2(sg, sg * kSeg, seg_len(sg), true);
  }

  if constexpr (GS > 0) {
    // the four fp32 partial tiles meet in LDS; wave 0 scales by S_x
    part[wave][lane] = __builtin_bit_cast(v4i, fsum);
    __syncthreads();
    if (wave == 0 && fac_dma) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the factor DMA (this wave's)
#pragma unroll
      for (int r = 0; r < 4; ++r) fbi[r] = fac[32 + 4 * lg + r];
    }
    if (wave == 0) {
      v4f t = __builtin_bit_cast(v4f, part[0][lane]);
#pragma unroll
      for (int w = 1; w < kWaves; ++w) t += __builtin_bit_cast(v4f, part[w][lane]);
      const int m = lr;
      if (m < M) {
        const float s_m = row_scale(m);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = n0 + lg * 4 + r;
          if (n < N) {
            float v = s_m * t[r];
            if (bias) v += fbi[r];
            store_out<YDT>(y, (size_t)m * N + n, v);
          }
        }
      }
    }
    return;
  }
  // ---- partial tiles and code sums meet in LDS; wave 0 applies the epilogue
  part[wave][lane] = acc;
  psum[wave][lane] = accs;
  __syncthreads();
  if (wave == 0) {
    if (fac_dma) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the factor DMA (this wave's)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        fsc[r] = fac[4 * lg + r];
        fzp[r] = fac[16 + 4 * lg + r];
        fbi[r] = fac[32 + 4 * lg + r];
      }
    }
    v4i t = part[0][lane], ts = psum[0][lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      t += part[w][lane];
      ts += psum[w][lane];
    }
    const int m = lr;
    if (m < M) {
      const float s_m = row_scale(m);
      const int r_m = ts[0];   // sum_k q_x[m, k]: every column of the all-ones product
      // The factors are first used here: the empty asm keeps their uses
      // (the zero point's conversion would otherwise be hoisted next to its
      // load, making the weight stream wait for the factor loads).
#pragma unroll
      for (int r = 0; r < 4; ++r) asm volatile("" : "+v"(fsc[r]), "+v"(fzp[r]), "+v"(fbi[r]));
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = n0 + lg * 4 + r;
        if (n < N) {
          const int a = t[r];
          if (acc_out) acc_out[(size_t)m * N + n] = a;
          const int c = a - (int)fzp[r] * r_m;
          float v = (s_m * fsc[r]) * (float)c;
          if (bias) v += fbi[r];
          store_out<YDT>(y, (size_t)m * N + n, v);
        }
      }
    }
  }
}

// ---- Decode on codes quantized beforehand (the row quantizer's codes, scales
// and code sums).  Past about ten tokens, quantizing every X row in every
// workgroup costs more vector work than the weight stream takes to arrive, so
// the rows are quantized once and this kernel only streams.  A workgroup owns
// 16 weight rows and its 4 waves split K; each wave copies its 1 KB share of
// the M code rows into its own LDS region (one contiguous 1 KB DMA per row),
// loads its share of the 16 weight rows straight into registers as the fused
// kernel does, and runs v_mfma_i32_16x16x64_i8 (weights as A, codes as B).
// (Staging the weights through LDS as well, one 1 KB DMA per row, took 7.4
// against ~5 us: the MFMAs then wait for both streams.)  Only the wave itself
// reads its region, so a wait on its own DMA replaces a barrier.  Rows past N
// (or M) repeat the last row and only feed outputs that are not stored;
// columns past K read past the row and their codes are masked to zero.
constexpr int kWPitch = kKW + 16;   // LDS bytes per row of a wave's K share (16-byte pad)

template <int YDT>
__global__ __launch_bounds__(kThreads, 1) void k_gemv_q8(const int8_t* __restrict__ xq,
                                                         const float* __restrict__ x_scale,
                                                         const int32_t* __restrict__ x_rowsum, int M, int K,
                                                         const int8_t* __restrict__ wq,
                                                         const float* __restrict__ w_scale,
                                                         const float* __restrict__ w_zp, int N,
                                                         const float* __restrict__ bias, void* __restrict__ y,
                                                         int32_t* __restrict__ acc_out, double y_inv) {
  __shared__ __attribute__((aligned(16))) uint8_t csm[kWaves][kRows * kWPitch];
  __shared__ v4i part[kWaves][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * kRows;
  // epilogue factors first (wave 0): register r of lane (lr, lg) is
  // D[n = n0 + 4 lg + r][m = lr]
  float fsc[4] = {0, 0, 0, 0}, fzp[4] = {0, 0, 0, 0}, fbi[4] = {0, 0, 0, 0};
  float s_m = 0.0f;
  int r_m = 0;
  const int m = lr;
  if (wave == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = n0 + 4 * lg + r;
      const int nc = n < N ? n : N - 1;
      fsc[r] = w_scale[nc];
      fzp[r] = w_zp[nc];
      fbi[r] = bias ? bias[nc] : 0.0f;
    }
    const int mc = m < M ? m : M - 1;
    s_m = x_scale[mc];
    r_m = x_rowsum[mc];
  }
  uint8_t* const cl = csm[wave];
  const int xr = lr < M ? lr : M - 1;     // code rows past M repeat the last: they feed unstored columns
  // weights straight into registers, as in the fused kernel: 16 loads of 16
  // bytes per lane (row n0 + lr, k-step s at s * 64 + 16 lg of the wave's
  // quarter), non-temporal, one offset per lane through a buffer resource;
  // past the segment they read the next row's bytes or the range check's
  // zeros, against zero codes
  const int wrow = (n0 + lr < N ? n0 + lr : N - 1);
  const __amdgpu_buffer_rsrc_t wres = byte_buffer(wq, (uint32_t)N * (uint32_t)K);
  v4i wv[kSteps];
  v4i acc = {0, 0, 0, 0};
  for (int k0 = 0; k0 < K; k0 += kSeg) {
    const int seg = (K - k0) < kSeg ? (K - k0) : kSeg;
    int c = wave * kKW + 16 * lane;
    c = c < seg ? c : seg - 16;                       // clamped; its codes are masked below
    if (k0 > 0) __builtin_amdgcn_s_waitcnt(kLgkmcnt0);   // this wave's reads of the last segment are done
    // the wave's 1 KB share of each of the M code rows first (contiguous 1 KB
    // per instruction), then the weights: the codes' wait leaves the weight
    // loads in flight
    const int mr = M < kRows ? M : kRows;
    for (int i = 0; i < mr; ++i) dma16((const uint8_t*)xq, (uint32_t)(i * K + k0 + c), cl + i * kWPitch);
    const uint32_t wbase = (uint32_t)(wrow * K + k0 + wave * kKW + lg * 16);
#pragma unroll
    for (int st = 0; st < kSteps; ++st) wv[st] = load16_nt(wres, wbase + st * 64);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kSteps) : "memory");
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const int o = st * 64 + lg * 16;
      v4i b = *(const v4i*)(cl + xr * kWPitch + o);
      if (seg != kSeg && wave * kKW + st * 64 + lg * 16 >= seg) b = v4i{0, 0, 0, 0};
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wv[st], b, acc, 0, 0, 0);
    }
  }
  part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && m < M) {
    v4i t = part[0][lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) t += part[w][lane];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = n0 + lg * 4 + r;
      if (n < N) {
        const int a = t[r];
        if (acc_out) acc_out[(size_t)m * N + n] = a;
        const int cc = a - (int)fzp[r] * r_m;
        if constexpr (YDT == DT_I8) {
          ((int8_t*)y)[(size_t)m * N + n] = (int8_t)requant_i8(s_m, fsc[r], cc, fbi[r], y_inv);
        } else {
          float v = (s_m * fsc[r]) * (float)cc;
          if (bias) v += fbi[r];
          store_out<YDT>(y, (size_t)m * N + n, v);
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
  const int m = (int)M, k = (int)K, n = (int)N;
  const bool one = K <= kSeg;
#define Q8_GEMV(YT)                                                                                     \
  (one ? (k_gemv_i8<DT, YT, true><<<grid, block, 0, st>>>(x, m, k, wq, ws, wz, n, bias, y, acc_out))   \
       : (k_gemv_i8<DT, YT, false><<<grid, block, 0, st>>>(x, m, k, wq, ws, wz, n, bias, y, acc_out)))
  switch (ydt) {
    case DT_F32: Q8_GEMV(DT_F32); break;
    case DT_F16: Q8_GEMV(DT_F16); break;
    default: Q8_GEMV(DT_BF16); break;
  }
#undef Q8_GEMV
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_q8(const int8_t* xq, const float* x_scale, const int32_t* x_rowsum, int64_t M, int64_t K,
                          const int8_t* wq, const float* w_scale, const float* w_zp, int64_t N, const float* bias,
                          void* y, int ydt, int32_t* acc_out, hipStream_t st, double y_inv) {
  dim3 grid((unsigned)((N + kRows - 1) / kRows)), block(kThreads);
  const int m = (int)M, k = (int)K, n = (int)N;
#define Q8_GEMV_Q8(YT) \
  k_gemv_q8<YT><<<grid, block, 0, st>>>(xq, x_scale, x_rowsum, m, k, wq, w_scale, w_zp, n, bias, y, acc_out, y_inv)
  switch (ydt) {
    case DT_I8: Q8_GEMV_Q8(DT_I8); break;
    case DT_F32: Q8_GEMV_Q8(DT_F32); break;
    case DT_F16: Q8_GEMV_Q8(DT_F16); break;
    default: Q8_GEMV_Q8(DT_BF16); break;
  }
#undef Q8_GEMV_Q8
  return hipGetLastError();
}

template <int DT, int GS>
hipError_t launch_grouped_dt(const void* x, int64_t M, int64_t K, const int8_t* wq, const float* ws,
                             const float* wz, int64_t N, const float* bias, void* y, int ydt, hipStream_t st) {
  dim3 grid((unsigned)((N + kRows - 1) / kRows)), block(kThreads);
  const int m = (int)M, k = (int)K, n = (int)N;
  const bool one = K <= kSeg;
#define Q8_GEMV_G(YT)                                                                                          \
  (one ? (k_gemv_i8<DT, YT, true, GS><<<grid, block, 0, st>>>(x, m, k, wq, ws, wz, n, bias, y, nullptr))       \
       : (k_gemv_i8<DT, YT, false, GS><<<grid, block, 0, st>>>(x, m, k, wq, ws, wz, n, bias, y, nullptr)))
  switch (ydt) {
    case DT_F32: Q8_GEMV_G(DT_F32); break;
    case DT_F16: Q8_GEMV_G(DT_F16); break;
    default: Q8_GEMV_G(DT_BF16); break;
  }
#undef Q8_GEMV_G
  return hipGetLastError();
}

template <int GS>
hipError_t launch_grouped_gs(const void* x, int xdt, int64_t M, int64_t K, const int8_t* wq, const float* ws,
                             const float* wz, int64_t N, const float* bias, void* y, int ydt, hipStream_t st) {
  switch (xdt) {
    case DT_F32: return launch_grouped_dt<DT_F32, GS>(x, M, K, wq, ws, wz, N, bias, y, ydt, st);
    case DT_F16: return launch_grouped_dt<DT_F16, GS>(x, M, K, wq, ws, wz, N, bias, y, ydt, st);
    default: return launch_grouped_dt<DT_BF16, GS>(x, M, K, wq, ws, wz, N, bias, y, ydt, st);
  }
}

hipError_t launch_gemv_i8_grouped(const void* x, int xdt, int64_t M, int64_t K, const int8_t* wq,
                                  const float* w_scale, const float* w_zp, int64_t group, int64_t N,
                                  const float* bias, void* y, int ydt, hipStream_t st) {
  if (group == 64) return launch_grouped_gs<64>(x, xdt, M, K, wq, w_scale, w_zp, N, bias, y, ydt, st);
  return launch_grouped_gs<128>(x, xdt, M, K, wq, w_scale, w_zp, N, bias, y, ydt, st);
}

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
