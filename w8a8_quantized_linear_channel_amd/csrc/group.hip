// Per-group asymmetric INT8 weights ("大模型量化技术概述" §2.2, granularity:
// groups of 64 to 128 parameters with their own scale and zero point; the
// lecture notes' granularity passage: per-group blocks).  Group j of row n is
// columns [j g, (j+1) g) of W; its scale S[j, n] and zero point Z[j, n] are
// stored group-major.  With per-token activation codes q_x, the layer is
//     y[m,n] = S_x[m] Sum_j S[j,n] (acc_j[m,n] - Z[j,n] gsum[j,m])  (+ b[n])
// where acc_j is the exact INT32 product over the group's columns and
// gsum[j, m] the sum of the activation codes over them.
//
//   k_quant_weight_grouped  one workgroup per row; the g/E lanes holding a
//                           group's 16-byte chunks take its min / max by
//                           lane shuffles, then every lane codes its chunk
//   k_gemv_group            decode, 11 <= M <= 16 (up to 10 tokens the fused
//                           decode kernel has a per-group mode): the on-codes
//                           decode layout
//                           (16 weight rows per workgroup, 4 waves splitting
//                           K, DMA of weight and code rows into LDS,
//                           v_mfma_i32_16x16x64_i8); after each group the
//                           INT32 tile is corrected by Z gsum exactly and
//                           added into fp32 with the group's scale
//   k_gemm_group            M > 16: a 128 x 128 tile of 8 waves (two per
//                           SIMD, each 64 x 32) on v_mfma_i32_32x32x32_i8,
//                           with the activations as the first operand so a
//                           lane's accumulators share one output column and
//                           one group scale.  Two accumulator sets alternate
//                           by group: the fold of one group (convert, fma
//                           with its scale into fp32) is interleaved with the
//                           MFMAs of the next.  The zero-point term
//                           -Sum_j S Z gsum is a rank-(K/g) fp32 product: one
//                           v_mfma_f32_32x32x2_f32 per pair of groups in the
//                           main loop, into the fp32 accumulators.  A group's
//                           S, Z and code sums for the whole tile come into
//                           LDS once, one 256-byte DMA per wave.
#include "q8_device.hpp"
#include "q8_group.hpp"

namespace q8 {
namespace {

// ------------------------------------------------------------------ weights
template <int DT>
__global__ __launch_bounds__(256) void k_quant_weight_grouped(const void* __restrict__ w, int64_t K, int64_t N,
                                                              int glanes, int8_t* __restrict__ wq,
                                                              float* __restrict__ w_scale,
                                                              float* __restrict__ w_zp) {
  constexpr int E = Chunk<DT>::kElems;
  constexpr int esz = DT == DT_F32 ? 4 : 2;
  const int64_t n = blockIdx.x;
  const int nch = (int)(K / E);
  const int64_t row = n * K;
  // chunk c is in group c / glanes; a group's chunks are glanes consecutive
  // lanes of one wave, all inside or all outside the row (K is a multiple of
  // the group size), so every lane of a group runs each iteration
  for (int c = threadIdx.x; c < nch; c += 256) {
    const v4i ch = *(const v4i*)((const char*)w + (row + (int64_t)c * E) * esz);
    float v[E];
    Chunk<DT>::decode(ch, v);
    float lo = 0.0f, hi = 0.0f;   // the range always contains 0
#pragma unroll
    for (int e = 0; e < E; ++e) {
      lo = fminf(lo, v[e]);
      hi = fmaxf(hi, v[e]);
    }
    for (int o = 1; o < glanes; o <<= 1) {
      lo = fminf(lo, __shfl_xor(lo, o, 64));
      hi = fmaxf(hi, __shfl_xor(hi, o, 64));
    }
    float s = (hi - lo) / 255.0f;
    s = s < kEps ? kEps : s;
    const float z = -128.0f - __builtin_rintf(lo / s);
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
    if constexpr (E == 8) *(v2i*)(wq + row + (int64_t)c * E) = v2i{(int)words[0], (int)words[1]};
    else *(uint32_t*)(wq + row + (int64_t)c * E) = words[0];
    if ((c & (glanes - 1)) == 0) {
      const int64_t j = c / glanes;
      w_scale[j * N + n] = s;
      w_zp[j * N + n] = z;
    }
  }
}

// ------------------------------------------------------------------ decode
constexpr int kRows = 16;              // weight rows per workgroup
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kSeg = 4096;             // K columns per segment
constexpr int kKW = kSeg / kWaves;     // columns of a segment per wave
constexpr int kSteps = kKW / 64;       // 64-column MFMA k-steps per wave per segment
constexpr int kWPitch = kKW + 16;      // LDS bytes per row of a wave's share (16-byte pad)

template <int YDT, int GS>
__global__ __launch_bounds__(kThreads, 1) void k_gemv_group(const int8_t* __restrict__ xq,
                                                            const float* __restrict__ x_scale,
                                                            const int32_t* __restrict__ gsum, int M, int K,
                                                            const int8_t* __restrict__ wq,
                                                            const float* __restrict__ w_scale,
                                                            const float* __restrict__ w_zp, int N,
                                                            const float* __restrict__ bias, void* __restrict__ y) {
  constexpr int SPG = GS / 64;         // k-steps per group
  constexpr int NG = kKW / GS;         // groups in a wave's share of a segment
  __shared__ __attribute__((aligned(16))) uint8_t csm[kWaves][kRows * kWPitch];
  __shared__ v4f part[kWaves][64];
  // groups of 128: each wave's 8 groups' scales and zero points for the 16
  // columns, one 1 KB DMA per wave and segment (group t's scales at
  // [32 t, 32 t + 16), its zero points at [32 t + 16, 32 t + 32))
  __shared__ __attribute__((aligned(16))) float gpar[GS == 128 ? kWaves : 1][256];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * kRows;
  const int G = K / GS;
  // register r of lane (lr, lg) is D[n = n0 + 4 lg + r][m = lr]
  const int m = lr;
  const int mc = m < M ? m : M - 1;
  int nc[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) nc[r] = n0 + 4 * lg + r < N ? n0 + 4 * lg + r : N - 1;
  // N a multiple of 4: the lane's columns n0 + 4 lg .. + 3 are one aligned
  // quad (clamped to the last quad past N; those outputs are not stored)
  const bool quad = (N & 3) == 0;
  const int q0 = n0 + 4 * lg < N ? n0 + 4 * lg : N - 4;
  uint8_t* const cl = csm[wave];
  const int xr = lr < M ? lr : M - 1;    // code rows past M repeat the last: they feed unstored columns
  const int wrow = (n0 + lr < N ? n0 + lr : N - 1);
  const __amdgpu_buffer_rsrc_t wres = byte_buffer(wq, (uint32_t)N * (uint32_t)K);
  v4i wv[kSteps];
  v4f f = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int k0 = 0; k0 < K; k0 += kSeg) {
    const int seg = (K - k0) < kSeg ? (K - k0) : kSeg;
    int c = wave * kKW + 16 * lane;
    c = c < seg ? c : seg - 16;                          // clamped; its codes are masked below
    if (k0 > 0) __builtin_amdgcn_s_waitcnt(kLgkmcnt0);   // this wave's reads of the last segment are done
    // the parameters of the share's groups first (groups past K are clamped
    // and not used), then the wave's 1 KB share of each code row, then the
    // weights straight into registers: the wait below leaves the weight
    // loads in flight
    // The parameters of the share's groups (groups past K are clamped and
    // not used).  With groups of 128, N a multiple of 4 and all 16 columns
    // present, by one DMA after the first four weight loads (gp); else by
    // vector loads here, ahead of the codes, under one branch around all the
    // groups' loads (a branch per group let the compiler's wait insertion
    // hold each group's loads until the previous group's had returned).
    const bool gp = GS == 128 && quad && n0 + kRows <= N;
    float ps[NG][4], pz[NG][4];
    int pg[NG];
    const int g0 = (k0 + wave * kKW) / GS;
    if (!gp) {
      if (quad) {   // the lane's four columns are one aligned 16-byte quad
#pragma unroll
        for (int t = 0; t < NG; ++t) {
          const int gi = g0 + t < G ? g0 + t : G - 1;
          const v4f sv = *(const v4f*)(w_scale + gi * N + q0), zv = *(const v4f*)(w_zp + gi * N + q0);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            ps[t][r] = sv[r];
            pz[t][r] = zv[r];
          }
        }
      } else {
#pragma unroll
        for (int t = 0; t < NG; ++t) {
          const int gi = g0 + t < G ? g0 + t : G - 1;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            ps[t][r] = w_scale[gi * N + nc[r]];
            pz[t][r] = w_zp[gi * N + nc[r]];
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < NG; ++t) pg[t] = gsum[(g0 + t < G ? g0 + t : G - 1) * M + mc];
    const int mr = M < kRows ? M : kRows;
    for (int i = 0; i < mr; ++i) dma16((const uint8_t*)xq, (uint32_t)(i * K + k0 + c), cl + i * kWPitch);
    // 16 loads of 16 bytes per lane (row n0 + lr, k-step s at s * 64 + 16 lg
    // of the wave's quarter), non-temporal, through a buffer resource; past
    // the segment they read the next row's bytes or the range check's zeros,
    // against zero codes
    const uint32_t wbase = (uint32_t)(wrow * K + k0 + wave * kKW + lg * 16);
#pragma unroll
    for (int st = 0; st < kSteps / 4; ++st) wv[st] = load16_nt(wres, wbase + st * 64);
    if constexpr (GS == 128) {
      if (gp) {
        // lane l: chunk l % 4 of the scales (bit 2 of l clear) or zero
        // points (set) of group g0 + l / 8
        const int t = lane >> 3, gi = g0 + t < G ? g0 + t : G - 1;
        const float* src = ((lane >> 2) & 1) ? w_zp : w_scale;
        dma16_ptr(src + (size_t)gi * N + n0 + 4 * (lane & 3), (uint8_t*)gpar[wave]);
      }
    }
#pragma unroll
    for (int st = kSteps / 4; st < kSteps; ++st) wv[st] = load16_nt(wres, wbase + st * 64);
    // the codes are in: everything but the weight loads (and the parameter
    // DMA among them)
    if (gp) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kSteps + 1) : "memory");
    else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kSteps) : "memory");
    if constexpr (GS == 128) {
      if (gp) {
        // the parameter DMA, followed by 12 weight loads
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kSteps - kSteps / 4) : "memory");
#pragma unroll
        for (int t = 0; t < NG; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            ps[t][r] = gpar[wave][32 * t + 4 * lg + r];
            pz[t][r] = gpar[wave][32 * t + 16 + 4 * lg + r];
          }
      }
    }
    v4i acc = {0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      const int o = s * 64 + lg * 16;
      v4i b = *(const v4i*)(cl + xr * kWPitch + o);
      if (seg != kSeg && wave * kKW + s * 64 + lg * 16 >= seg) b = v4i{0, 0, 0, 0};
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wv[s], b, acc, 0, 0, 0);
      if ((s + 1) % SPG == 0) {
        const int t = s / SPG;
        if (wave * kKW + t * GS < seg) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int cc = acc[r] - (int)pz[t][r] * pg[t];   // exact: |cc| < 2^24
            f[r] = fmaf(ps[t][r], (float)cc, f[r]);
          }
        }
        acc = v4i{0, 0, 0, 0};
      }
    }
  }
  part[wave][lane] = f;
  __syncthreads();
  if (wave == 0 && m < M) {
    v4f t = part[0][lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) t += part[w][lane];
    const float sx = x_scale[m];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = n0 + lg * 4 + r;
      if (n < N) {
        float v = sx * t[r];
        if (bias) v += bias[n];
        store_out<YDT>(y, (size_t)m * N + n, v);
      }
    }
  }
}

// ------------------------------------------------------------------ GEMM
namespace gg {
constexpr int kBK = 64;                         // bytes of K per stage
constexpr int KS = kBK / 32;                    // k-steps per stage
constexpr int kStages = 4;
constexpr int kMetaSlot = 2048;                 // per stage: the group's S, Z (128 columns), code sums (128 rows), spare
constexpr int kRowsPerDma = 16;                 // one 1 KB DMA = 16 rows of 64 bytes
constexpr int kXcds = 8, kGroupM = 4;
}  // namespace gg

// A BM x BN tile of NW waves in a (NW / WN) x WN grid, 32 x 32 fragments.
// DB: two accumulator sets (the fold of a group overlaps the next group's
// MFMAs); else one set, folded between the groups.
template <int BM_, int BN_, int NW_, int WN_, bool DB_ = true>
struct GTile {
  static constexpr bool DB = DB_;
  static constexpr int BM = BM_, BN = BN_, NW = NW_, NT = 64 * NW_, WN = WN_, WM = NW_ / WN_;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr int ALOADS = BM * (gg::kBK / 16) / NT, BLOADS = BN * (gg::kBK / 16) / NT;
  // DMA per wave and stage: A rows and B rows; the first stage of a group
  // adds one DMA of the group's parameters
  static constexpr int AB = ALOADS + BLOADS;
  static constexpr int kStageBytes = (BM + BN) * gg::kBK;
  static_assert(ALOADS >= 1 && BLOADS >= 1 && FM >= 1 && FN >= 1 && (TN == 32 || TN == 64), "tile shape");
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * gg::kBK + ((chunk ^ ((row >> 2) & 3)) << 4); }
// v_mfma_i32_32x32x32_i8 operand of lane l: row (base + l % 32), logical
// 16-byte chunk 2 ks + l / 32 of the row, found at its swizzled position
__device__ __forceinline__ int lane_off(int lane) { return ((lane >> 5) ^ ((lane >> 2) & 3)) << 4; }
__device__ __forceinline__ int out_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// global_load_lds_dword: 64 lanes x 4 bytes from gbase + voff into 256 bytes
// of LDS at `lds` (lane l at lds + 4 l), counted by vmcnt like dma16.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma4(const uint8_t* gbase, uint32_t voff, uint8_t* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(lptr_t)lds;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :
               : "s"(m0), "v"(voff), "s"(gbase)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(n) for a uniform n in 0..N (the count must be an immediate)
template <int N>
__device__ __forceinline__ void vm_wait_upto(int n) {
  if constexpr (N == 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    if (n >= N) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
    else vm_wait_upto<N - 1>(n);
  }
}

// XCD-contiguous renumbering, then kGroupM tile-rows per L2 group
__device__ __forceinline__ void group_tile_coords(int ntm, int ntn, int& tm, int& tn) {
  const int T = ntm * ntn;
  const int b = blockIdx.x;
  const int q = T / gg::kXcds, r = T % gg::kXcds;
  const int x = b % gg::kXcds, i = b / gg::kXcds;
  const int bp = x * q + (x < r ? x : r) + i;
  const int per_group = gg::kGroupM * ntn;
  const int group = bp / per_group;
  const int first_m = group * gg::kGroupM;
  const int gsize = (ntm - first_m) < gg::kGroupM ? (ntm - first_m) : gg::kGroupM;
  const int inner = bp - group * per_group;
  tm = first_m + inner % gsize;
  tn = inner / gsize;
}

template <class TL, int YDT, int GS>
__global__ __launch_bounds__(TL::NT, 1) void k_gemm_group(const int8_t* __restrict__ xq,
                                                         const float* __restrict__ x_scale,
                                                         const int32_t* __restrict__ gsum, int M, int K,
                                                         const int8_t* __restrict__ wq,
                                                         const float* __restrict__ w_scale,
                                                         const float* __restrict__ w_zp, int N,
                                                         const float* __restrict__ bias, void* __restrict__ y) {
  using namespace gg;
  constexpr int BM = TL::BM, BN = TL::BN, NW = TL::NW, NT = TL::NT, WN = TL::WN;
  constexpr int TM = TL::TM, TN = TL::TN, FM = TL::FM, FN = TL::FN;
  constexpr int ALOADS = TL::ALOADS, BLOADS = TL::BLOADS, AB = TL::AB;
  constexpr int kStageBytes = TL::kStageBytes;
  constexpr int SPG = GS / kBK;   // stages per group (1 or 2)
  __shared__ __attribute__((aligned(16))) uint8_t smem[kStages * kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t meta[kStages * kMetaSlot];
  __shared__ float f_sx[BM];
  uint8_t* const sa0 = smem;
  uint8_t* const sb0 = smem + BM * kBK;
  uint8_t* const sa1 = smem + kStageBytes;
  uint8_t* const sb1 = sa1 + BM * kBK;
  uint8_t* const sa2 = smem + 2 * kStageBytes;
  uint8_t* const sb2 = sa2 + BM * kBK;
  uint8_t* const sa3 = smem + 3 * kStageBytes;
  uint8_t* const sb3 = sa3 + BM * kBK;

  int tm, tn;
  group_tile_coords((M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int G = K / GS;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int swave = __builtin_amdgcn_readfirstlane(wave);
  const int wm = wave / WN, wn = wave % WN;
  // the lane's output column in fragment column jj (one per lane: the
  // activations are the MFMA's first operand, so D[m][n] has n = l % 32)
  int ncol[FN], ncl[FN];
  float bn[FN];
#pragma unroll
  for (int jj = 0; jj < FN; ++jj) {
    ncol[jj] = n0 + wn * TN + jj * 32 + (lane & 31);
    ncl[jj] = ncol[jj] < N ? ncol[jj] : N - 1;
    bn[jj] = bias ? bias[ncl[jj]] : 0.0f;
  }
  // row scales, read after the main loop's barriers
#pragma unroll
  for (int u = 0; u < (BM + NT - 1) / NT; ++u) {
    const int t = tid + u * NT;
    if (t < BM) f_sx[t] = x_scale[m0 + t < M ? m0 + t : M - 1];
  }

  // ---- DMA: lane l lands at row l / 4, physical chunk l % 4 of a 16-row
  // block, which holds logical chunk (l % 4) ^ ((row >> 2) & 3); rows past M
  // (or N) re-read the last row and only feed outputs that are not stored.
  const int lrow = lane >> 2;
  const int lchunk = (lane & 3) ^ ((lrow >> 2) & 3);
  uint32_t aoff[ALOADS], boff[BLOADS];
#pragma unroll
  for (int j = 0; j < ALOADS; ++j) {
    int gm = m0 + (j * NW + swave) * kRowsPerDma + lrow;
    gm = gm < M ? gm : M - 1;
    aoff[j] = (uint32_t)(gm * K + lchunk * 16);
  }
#pragma unroll
  for (int j = 0; j < BLOADS; ++j) {
    int gn = n0 + (j * NW + swave) * kRowsPerDma + lrow;
    gn = gn < N ? gn : N - 1;
    boff[j] = (uint32_t)(gn * K + lchunk * 16);
  }
  const int nfull = K / kBK;   // K is a multiple of GS, hence of 64
  // The group's parameters for the whole tile, once per group, into the
  // stage's meta slot: one 256-byte DMA per wave.  Waves 0, 1: S[j, n] of the
  // tile's 128 columns (bytes 0..511 of the slot); 2, 3: Z[j, n] (512..1023);
  // 4, 5: the code sums gsum[j, m] of its 128 rows (1024..1535); 6, 7 a second
  // copy of S into the spare bytes, so that every wave issues the same number
  // of DMAs and one vmcnt fits all.
  static_assert(BM == 128 && BN == 128 && NW == 8, "eight 64-entry parameter DMAs per group");
  const int mk = swave >> 1, mh = swave & 1;
  const uint8_t* mbase;
  int mstride, mlds, mix;
  if (mk == 2) {
    mix = m0 + mh * 64 + lane;
    mix = mix < M ? mix : M - 1;
    mbase = (const uint8_t*)gsum;
    mstride = M;
  } else {
    mix = n0 + mh * 64 + lane;
    mix = mix < N ? mix : N - 1;
    mbase = (const uint8_t*)(mk == 1 ? w_zp : w_scale);
    mstride = N;
  }
  mlds = mk * 512 + mh * 256;
  const uint32_t moff = (uint32_t)mix * 4u;
  auto meta_at = [&](int s) __attribute__((always_inline)) { return meta + (s & (kStages - 1)) * kMetaSlot; };
  auto dma_one = [&](int k, uint8_t* sa, uint8_t* sb, int s) __attribute__((always_inline)) {
    if (k < ALOADS)
      dma16((const uint8_t*)xq + s * kBK, aoff[k], sa + (k * NW + swave) * kRowsPerDma * kBK);
    else if (k < AB)
      dma16((const uint8_t*)wq + s * kBK, boff[k - ALOADS], sb + ((k - ALOADS) * NW + swave) * kRowsPerDma * kBK);
    else
      dma4(mbase, moff + (uint32_t)((s / SPG) * mstride) * 4u, meta_at(s) + mlds);
  };
  // DMA instructions of stage t (0 past the last stage)
  auto loads_of = [&](int t) __attribute__((always_inline)) { return t < nfull ? AB + (t % SPG == 0) : 0; };
  auto dma = [&](uint8_t* sa, uint8_t* sb, int s) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < AB; ++k) dma_one(k, sa, sb, s);
    if (s % SPG == 0) dma_one(AB, sa, sb, s);
  };

  // fp32 accumulators; the zero-point term -Sum_j (S Z)[j, n] gsum[j, m]
  // enters in the main loop, two groups per v_mfma_f32_32x32x2_f32 (lane l:
  // A[m = l % 32][k = l / 32], B[k][n = l % 32]), k = 0 the earlier group
  v16f f[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int jj = 0; jj < FN; ++jj) f[i][jj] = v16f{};
  if (nfull > 0) dma(sa0, sb0, 0);
  if (nfull > 1) dma(sa1, sb1, 1);
  if (nfull > 2) dma(sa2, sb2, 2);
  // the earlier group of the current pair: its code sums and -S Z
  float gprev[FM], pprev[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) gprev[i] = 0.0f;
#pragma unroll
  for (int jj = 0; jj < FN; ++jj) pprev[jj] = 0.0f;

  using Acc = v16i;
  constexpr int NSET = TL::DB ? 2 : 1;
  Acc acc[NSET][FM][FN];
#pragma unroll
  for (int h = 0; h < NSET; ++h)
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int jj = 0; jj < FN; ++jj) acc[h][i][jj] = Acc{};
  float sgrp[2][FN];   // the scales of the group in each accumulator set
#pragma unroll
  for (int jj = 0; jj < FN; ++jj) sgrp[0][jj] = sgrp[1][jj] = 0.0f;

  const int arow = (wm * TM + (lane & 31)) * kBK;
  const int brow = (wn * TN + (lane & 31)) * kBK;
  const int loff = lane_off(lane);
  v4i fa[2][FM], fb[2][FN];
  auto load_frag = [&](auto SET, int fi, const uint8_t* As, const uint8_t* Bs, int ks) __attribute__((always_inline)) {
    constexpr int st = decltype(SET)::value;
    if (fi < FM) fa[st][fi] = *(const v4i*)(As + arow + fi * 32 * kBK + (loff ^ (ks << 5)));
    else fb[st][fi - FM] = *(const v4i*)(Bs + brow + (fi - FM) * 32 * kBK + (loff ^ (ks << 5)));
  };
  auto load_frags = [&](auto SET, const uint8_t* As, const uint8_t* Bs, int ks) __attribute__((always_inline)) {
#pragma unroll
    for (int fi = 0; fi < FM + FN; ++fi) load_frag(SET, fi, As, Bs, ks);
  };
  // fold part q (0 .. 2 FM FN - 1) of accumulator set H: 8 elements of
  // fragment q / 2
  auto fold = [&](auto HC, int q) __attribute__((always_inline)) {
    constexpr int H = decltype(HC)::value;
    const int fi = q >> 1, i = fi / FN, jj = fi % FN, r0 = (q & 1) * 8;
#pragma unroll
    for (int r = 0; r < 8; ++r)
      f[i][jj][r0 + r] = fmaf(sgrp[H][jj], (float)acc[H][i][jj][r0 + r], f[i][jj][r0 + r]);
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using T = std::true_type;
  using F = std::false_type;
  constexpr int NM = FM * FN;   // MFMAs per k-step; a stage (KS = 2) has 2 NM slots for 2 NM fold parts
  static_assert(KS == 2, "a stage is two k-steps of the 32x32x32 MFMA");
  // One k-step's MFMAs on fragment set CUR into accumulator set H, with the
  // LDS reads of the next fragments (pf), DMA instructions of a later stage
  // (dm) and fold parts of the other accumulator set (fl) spread between
  // them; ZERO: the group's first k-step, whose MFMAs start from 0.
  auto step = [&](auto CUR, auto NXT, auto HC, auto ZERO, auto MD, bool fl, int fq, bool pf, bool dm,
                  const uint8_t* xa, const uint8_t* xb, int xks, uint8_t* da, uint8_t* db,
                  int ds) __attribute__((always_inline)) {
    constexpr int cs = decltype(CUR)::value;
    constexpr int H = decltype(HC)::value;
    constexpr int NF = FM + FN, NL = AB + (decltype(MD)::value ? 1 : 0);
#pragma unroll
    for (int t = 0; t < NM; ++t) {
      const int i = t / FN, jj = t % FN;
      acc[H][i][jj] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
          fa[cs][i], fb[cs][jj], decltype(ZERO)::value ? Acc{} : acc[H][i][jj], 0, 0, 0);
      if constexpr (TL::DB) {
        if (fl) {
          using O = std::integral_constant<int, H ^ 1>;
          fold(O{}, fq + t);
        }
      }
      if (pf) {
#pragma unroll
        for (int fi = (t * NF + NM - 1) / NM; fi < ((t + 1) * NF + NM - 1) / NM; ++fi) load_frag(NXT, fi, xa, xb, xks);
      }
      if (dm) {
#pragma unroll
        for (int k = (t * NL + NM - 1) / NM; k < ((t + 1) * NL + NM - 1) / NM; ++k) dma_one(k, da, db, ds);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Stage s complete: the DMAs of the (at most two) stages issued after it
  // may still be in flight.  In the steady state one of every two
  // consecutive stages opens a group when SPG = 2, both when SPG = 1.
  auto wait_stage = [&](int s, bool steady) __attribute__((always_inline)) {
    if (steady) vm_wait_upto<2 * AB + 2 / SPG>(2 * AB + 2 / SPG);
    else vm_wait_upto<2 * AB + 2>(loads_of(s + 1) + loads_of(s + 2));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // One stage (KS = 2 k-steps) whose first k-step's fragments are in register
  // set 0 (KS is even, so every stage starts in set 0).  HC: accumulator set
  // of the stage's group; FIRST: the stage opens its group (its MFMAs start
  // from 0, it reads the group's scales, and it folds the other set, which
  // holds the previous group).
  auto stage = [&](auto STEADY, auto HC, auto FIRST, int s, uint8_t* ca, uint8_t* cb, const uint8_t* xa,
                   const uint8_t* xb) __attribute__((always_inline)) {
    constexpr int PAR = decltype(HC)::value;   // the group's parity
    constexpr int H = TL::DB ? PAR : 0;        // its accumulator set
    constexpr bool first = decltype(FIRST)::value;
    constexpr bool steady = decltype(STEADY)::value;
    if constexpr (!TL::DB) {
      // one accumulator set: fold the previous group before this one starts
      if (first) {
#pragma unroll
        for (int q = 0; q < 2 * NM; ++q) fold(S0{}, q);
      }
    }
    float zc[FN], gc[FM];
    if (first) {
      const uint8_t* mt = meta_at(s);
#pragma unroll
      for (int jj = 0; jj < FN; ++jj) {
        const int c = wn * TN + jj * 32 + (lane & 31);
        sgrp[H][jj] = *(const float*)(mt + 4 * c);
        zc[jj] = *(const float*)(mt + 512 + 4 * c);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) gc[i] = (float)*(const int*)(mt + 1024 + 4 * (wm * TM + i * 32 + (lane & 31)));
    }
    using HS = std::integral_constant<int, H>;
    using Z = std::integral_constant<bool, first>;
    step(S0{}, S1{}, HS{}, Z{}, F{}, first, 0, true, false, ca, cb, 1, ca, cb, 0);
    __builtin_amdgcn_s_waitcnt(kLgkmcnt0);
    const bool nxt = steady || s + 1 < nfull;
    const bool ahead = steady || s + 4 < nfull;
    if (nxt) wait_stage(s + 1, steady);
    // the stage DMA'd here, s + 4, opens a group exactly when s does
    step(S1{}, S0{}, HS{}, F{}, FIRST, first, NM, nxt, ahead, xa, xb, 0, ca, cb, s + 4);
    if (first) {
      // the group's zero-point term, after this stage's fold parts: groups
      // alternate between the two k of the MFMA (H is the group's parity)
      float pc[FN];
#pragma unroll
      for (int jj = 0; jj < FN; ++jj) pc[jj] = -(sgrp[H][jj] * zc[jj]);
      if constexpr (PAR == 1) {
        const bool lo = lane < 32;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int jj = 0; jj < FN; ++jj)
            f[i][jj] = __builtin_amdgcn_mfma_f32_32x32x2f32(lo ? gprev[i] : gc[i], lo ? pprev[jj] : pc[jj], f[i][jj],
                                                            0, 0, 0);
      } else {
#pragma unroll
        for (int i = 0; i < FM; ++i) gprev[i] = gc[i];
#pragma unroll
        for (int jj = 0; jj < FN; ++jj) pprev[jj] = pc[jj];
      }
    }
  };
  // accumulator set and group opening of stage offset o in a 4-stage block
  using H0 = std::integral_constant<int, 0>;
  using H1 = std::integral_constant<int, (1 / SPG) & 1>;
  using H2 = std::integral_constant<int, (2 / SPG) & 1>;
  using H3 = std::integral_constant<int, (3 / SPG) & 1>;
  using F1 = std::integral_constant<bool, 1 % SPG == 0>;
  using F3 = std::integral_constant<bool, 3 % SPG == 0>;

  if (nfull > 0) {
    wait_stage(0, false);
    if (nfull > 3) dma(sa3, sb3, 3);
    load_frags(S0{}, sa0, sb0, 0);
  }
  int kt = 0;
  for (; kt + 8 <= nfull; kt += 4) {
    stage(T{}, H0{}, T{}, kt, sa0, sb0, sa1, sb1);
    stage(T{}, H1{}, F1{}, kt + 1, sa1, sb1, sa2, sb2);
    stage(T{}, H2{}, T{}, kt + 2, sa2, sb2, sa3, sb3);
    stage(T{}, H3{}, F3{}, kt + 3, sa3, sb3, sa0, sb0);
  }
  if (kt + 4 <= nfull) {
    stage(F{}, H0{}, T{}, kt, sa0, sb0, sa1, sb1);
    stage(F{}, H1{}, F1{}, kt + 1, sa1, sb1, sa2, sb2);
    stage(F{}, H2{}, T{}, kt + 2, sa2, sb2, sa3, sb3);
    stage(F{}, H3{}, F3{}, kt + 3, sa3, sb3, sa0, sb0);
    kt += 4;
  }
  if (kt < nfull) stage(F{}, H0{}, T{}, kt, sa0, sb0, sa1, sb1);
  if (kt + 1 < nfull) stage(F{}, H1{}, F1{}, kt + 1, sa1, sb1, sa2, sb2);
  if (kt + 2 < nfull) stage(F{}, H2{}, T{}, kt + 2, sa2, sb2, sa3, sb3);
  // the last group's fold
  if constexpr (TL::DB) {
    if (((nfull / SPG - 1) & 1) == 0) {
#pragma unroll
      for (int q = 0; q < 2 * NM; ++q) fold(H0{}, q);
    } else {
#pragma unroll
      for (int q = 0; q < 2 * NM; ++q) fold(S1{}, q);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 2 * NM; ++q) fold(H0{}, q);
  }
  if (G & 1) {   // the last group had no partner: k = 1 is zero
    const bool lo = lane < 32;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int jj = 0; jj < FN; ++jj)
        f[i][jj] = __builtin_amdgcn_mfma_f32_32x32x2f32(lo ? gprev[i] : 0.0f, lo ? pprev[jj] : 0.0f, f[i][jj], 0, 0, 0);
  }

  // ---- epilogue: y = S_x[m] f (+ b[n]) in the output type, one 32-row slab
  // of the wave tile at a time through LDS (the main loop's arena): a lane
  // holds one column of 16 rows, the readback gives each lane 16 bytes of one
  // row, which leave as one store.
  constexpr int ES = YDT == DT_F32 ? 4 : 2;
  constexpr int kRowB = TN * ES;                 // bytes of a wave-tile row
  constexpr int kPitchE = kRowB + 16;            // the two half-waves' rows fall in different banks
  constexpr int LPR = kRowB / 16;                // readback lanes per row
  constexpr int RPI = 64 / LPR;                  // rows per readback instruction
  static_assert(NW * 32 * kPitchE <= kStages * kStageBytes, "epilogue staging does not fit");
  __syncthreads();                               // every wave's main-loop LDS reads are done
  uint8_t* const stg = smem + wave * 32 * kPitchE;
  const bool vec = (N % (16 / ES)) == 0;         // 16-byte groups of a row start aligned
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int jj = 0; jj < FN; ++jj)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rl = out_row(r, lane);
        float v = f_sx[wm * TM + i * 32 + rl] * f[i][jj][r];
        if (bias) v += bn[jj];
        uint8_t* p = stg + rl * kPitchE + (jj * 32 + (lane & 31)) * ES;
        if constexpr (YDT == DT_F32) *(float*)p = v;
        else if constexpr (YDT == DT_F16) *(uint16_t*)p = f32_to_f16(v);
        else *(uint16_t*)p = f32_to_bf16(v);
      }
    // the wave's own staging writes precede these reads (LDS is in order)
#pragma unroll
    for (int t = 0; t < 32 / RPI; ++t) {
      const int row = t * RPI + lane / LPR;
      const int cb = (lane % LPR) * 16;
      const v4i val = *(const v4i*)(stg + row * kPitchE + cb);
      const int m = m0 + wm * TM + i * 32 + row;
      const int n = n0 + wn * TN + cb / ES;
      if (m < M) {
        uint8_t* dst = (uint8_t*)y + ((size_t)m * N + n) * ES;
        if (vec && n + 16 / ES <= N) {
          *(v4i*)dst = val;
        } else {
#pragma unroll
          for (int e = 0; e < 16 / ES; ++e)
            if (n + e < N) {
              if constexpr (ES == 4) ((int*)dst)[e] = val[e];
              else ((uint16_t*)dst)[e] = (uint16_t)((uint32_t)val[e >> 1] >> (16 * (e & 1)));
            }
        }
      }
    }
  }
}

// the tile the launcher uses
using GemmTile = GTile<128, 128, 8, 4>;

template <int GS>
hipError_t gemv_gs(const int8_t* xq, const float* xs, const int32_t* gs, int64_t M, int64_t K, const int8_t* wq,
                   const float* ws, const float* wz, int64_t N, const float* bias, void* y, int ydt, hipStream_t st) {
  dim3 grid((unsigned)((N + kRows - 1) / kRows)), block(kThreads);
  const int m = (int)M, k = (int)K, n = (int)N;
  switch (ydt) {
    case DT_F32: k_gemv_group<DT_F32, GS><<<grid, block, 0, st>>>(xq, xs, gs, m, k, wq, ws, wz, n, bias, y); break;
    case DT_F16: k_gemv_group<DT_F16, GS><<<grid, block, 0, st>>>(xq, xs, gs, m, k, wq, ws, wz, n, bias, y); break;
    default: k_gemv_group<DT_BF16, GS><<<grid, block, 0, st>>>(xq, xs, gs, m, k, wq, ws, wz, n, bias, y); break;
  }
  return hipGetLastError();
}

template <int GS>
hipError_t gemm_gs(const int8_t* xq, const float* xs, const int32_t* gs, int64_t M, int64_t K, const int8_t* wq,
                   const float* ws, const float* wz, int64_t N, const float* bias, void* y, int ydt, hipStream_t st) {
  using TL = GemmTile;
  const unsigned tiles = (unsigned)(((M + TL::BM - 1) / TL::BM) * ((N + TL::BN - 1) / TL::BN));
  const int m = (int)M, k = (int)K, n = (int)N;
  switch (ydt) {
    case DT_F32: k_gemm_group<TL, DT_F32, GS><<<tiles, TL::NT, 0, st>>>(xq, xs, gs, m, k, wq, ws, wz, n, bias, y); break;
    case DT_F16: k_gemm_group<TL, DT_F16, GS><<<tiles, TL::NT, 0, st>>>(xq, xs, gs, m, k, wq, ws, wz, n, bias, y); break;
    default: k_gemm_group<TL, DT_BF16, GS><<<tiles, TL::NT, 0, st>>>(xq, xs, gs, m, k, wq, ws, wz, n, bias, y); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_weight_grouped(const void* w, int dt, int64_t N, int64_t K, int64_t group, int8_t* wq,
                                       float* w_scale, float* w_zp, hipStream_t st) {
  dim3 grid((unsigned)N), block(256);
  switch (dt) {
    case DT_F32:
      k_quant_weight_grouped<DT_F32><<<grid, block, 0, st>>>(w, K, N, (int)(group / 4), wq, w_scale, w_zp);
      break;
    case DT_F16:
      k_quant_weight_grouped<DT_F16><<<grid, block, 0, st>>>(w, K, N, (int)(group / 8), wq, w_scale, w_zp);
      break;
    default:
      k_quant_weight_grouped<DT_BF16><<<grid, block, 0, st>>>(w, K, N, (int)(group / 8), wq, w_scale, w_zp);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_gemv_group(const int8_t* xq, const float* x_scale, const int32_t* gsum, int64_t M, int64_t K,
                             const int8_t* wq, const float* w_scale, const float* w_zp, int64_t group, int64_t N,
                             const float* bias, void* y, int ydt, hipStream_t st) {
  if (group == 64) return gemv_gs<64>(xq, x_scale, gsum, M, K, wq, w_scale, w_zp, N, bias, y, ydt, st);
  return gemv_gs<128>(xq, x_scale, gsum, M, K, wq, w_scale, w_zp, N, bias, y, ydt, st);
}

hipError_t launch_gemm_group(const int8_t* xq, const float* x_scale, const int32_t* gsum, int64_t M, int64_t K,
                             const int8_t* wq, const float* w_scale, const float* w_zp, int64_t group, int64_t N,
                             const float* bias, void* y, int ydt, hipStream_t st) {
  if (group == 64) return gemm_gs<64>(xq, x_scale, gsum, M, K, wq, w_scale, w_zp, N, bias, y, ydt, st);
  return gemm_gs<128>(xq, x_scale, gsum, M, K, wq, w_scale, w_zp, N, bias, y, ydt, st);
}

}  // namespace q8
