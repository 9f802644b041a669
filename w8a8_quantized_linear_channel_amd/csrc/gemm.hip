// MFMA GEMM for the quantized linear layer, Y = epilogue(A . B^T), with both
// operands K-contiguous 1-byte codes ("NT" layout): A = activation codes
// [M, K], B = weight codes [N, K].
//
//   GEMM_INT8         v_mfma_i32_32x32x32_i8, exact INT32 accumulation, then
//                     y = S_a[m] S_b[n] (acc - Z_b[n] rowsum_a[m]) (+ bias)
//                     (the 32x32x32 shape: on gfx950 the 16x16x64 int8 MFMA
//                     issues at half its rate)
//   GEMM_INT8_DECOMP  as GEMM_INT8, then the LLM.int8 outlier flow is added
//                     with v_mfma_f32_32x32x16_f16 on top of the dequantized
//                     accumulator: y += X[:, O] . fp16(S_b (Wq[:, O] - Z_b))^T
//   GEMM_FP8          v_mfma_f32_32x32x64_f8f6f4 on e4m3 codes, fp32
//                     accumulation, y = S_a[m] S_b[n] acc (+ bias)
//
// Tiling: a workgroup of 4 waves (2 x 2) owns a BM x BN output tile; each wave
// owns (BM/2) x (BN/2) built from 32 x 32 MFMA fragments.  K advances 64
// bytes per stage.  Four LDS buffers hold four stages, filled by
// global_load_lds_dwordx4 (global -> LDS without registers) three stages
// ahead of the MFMAs, so a stage's loads have three stages of compute to
// arrive.  Within a stage the B fragments of k-step s+1 are read from LDS while
// the MFMAs of k-step s run, and each A fragment is re-read right after its
// last use.
//
// LDS layout: row-major 64-byte rows (one row of the tile, one stage of K),
// the 16-byte chunk c of row r stored at chunk position c ^ ((r >> 1) & 3).
// A fragment read has rows 0..7 of one logical chunk in one LDS cycle; even
// and odd rows fall in different halves of the banks and the XOR spreads the
// four row pairs over the four bank groups of each half.  The DMA writes 64
// consecutive 16-byte slots per wave instruction, so the swizzle is applied
// on the global side: each lane fetches the chunk that belongs at its slot.
//
// Workgroups are renumbered so consecutive tiles land on the same XCD (the
// dispatcher deals workgroups round-robin over the 8 XCDs) and, within an
// XCD, 4 tile-rows share each weight tile in L2.
//
// Indices are 32-bit: the host guarantees M*K, N*K and M*N are below 2^31.
#include "q8_device.hpp"
#include "q8_kernels.hpp"

namespace q8 {
namespace {

typedef __attribute__((address_space(1))) void* gptr_t;   // global (DMA source)
typedef __attribute__((address_space(3))) void* lptr_t;   // LDS (DMA destination)

constexpr int kBK = 64;             // bytes of K per stage
constexpr int kStages = 4;          // LDS buffers (prefetch distance kStages - 1)
constexpr int kThreads = 256;       // 4 waves
constexpr int kGroupM = 4;          // tile-rows per L2 group
constexpr int kXcds = 8;

__device__ __forceinline__ int swz(int row, int chunk) { return row * kBK + ((chunk ^ ((row >> 1) & 3)) << 4); }

// One MFMA shape.  A fragment row is (base multiple of 32) + lane % 32, so
// ((row >> 1) & 3) == ((lane >> 1) & 3) and the swizzled byte offset of the
// lane's operand inside its LDS row is lane_off(lane) XOR a per-k-step constant.
// A and B fragments use the same lane -> k mapping, so each instruction sums
// over exactly the k bytes of its step whatever order the hardware uses.
struct MmaI8 {                       // v_mfma_i32_32x32x32_i8
  static constexpr int KSTEP = 32, NR = 16;
  using Op = v4i;
  using Acc = v16i;
  // lane l: 16-byte logical chunk 2*ks + l/32 of its row
  __device__ static int lane_off(int lane) { return ((lane >> 5) ^ ((lane >> 1) & 3)) << 4; }
  __device__ static Op load(const uint8_t* row, int off, int ks) {
    return *(const v4i*)(row + (off ^ (ks << 5)));
  }
  __device__ static Acc mma(const Op& a, const Op& b, const Acc& c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
  }
};
struct MmaF8 {                       // v_mfma_f32_32x32x64_f8f6f4, both operands e4m3
  static constexpr int KSTEP = 64, NR = 16;
  using Op = v8i;
  using Acc = v16f;
  // lane l: logical chunks 4*ks + 2*(l/32) + {0, 1} of its row
  __device__ static int lane_off(int lane) { return ((2 * (lane >> 5)) ^ ((lane >> 1) & 3)) << 4; }
  __device__ static Op load(const uint8_t* row, int off, int ks) {
    const v4i lo = *(const v4i*)(row + (off ^ (ks << 6)));
    const v4i hi = *(const v4i*)(row + ((off ^ 16) ^ (ks << 6)));
    return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  __device__ static Acc mma(const Op& a, const Op& b, const Acc& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
  }
};
// 32 x 32 output fragment layout (all 32x32 MFMAs): register r of lane l is
// row 8*(r/4) + 4*(l/32) + r%4, column l%32.
__device__ __forceinline__ int out_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

template <int BM, int BN>
struct Tile {
  static constexpr int TM = BM / 2, TN = BN / 2;            // wave tile
  static constexpr int FM = TM / 32, FN = TN / 32;          // 32x32 fragments per wave
  static constexpr int ALOADS = BM * (kBK / 16) / kThreads;   // 16-byte chunks per thread
  static constexpr int BLOADS = BN * (kBK / 16) / kThreads;
  static constexpr int LOADS = ALOADS + BLOADS;               // DMA instructions per wave per stage
  static_assert(ALOADS >= 1 && BLOADS >= 1 && FM >= 1 && FN >= 1, "tile too small");
};

// Tile coordinates of this workgroup: XCD-contiguous renumbering, then
// grouped (kGroupM tile-rows) column-major order inside a group.
__device__ __forceinline__ void tile_coords(int ntm, int ntn, int& tm, int& tn) {
  const int T = ntm * ntn;
  const int b = blockIdx.x;
  const int q = T / kXcds, r = T % kXcds;
  const int x = b % kXcds, i = b / kXcds;
  const int bp = x * q + (x < r ? x : r) + i;
  const int per_group = kGroupM * ntn;
  const int group = bp / per_group;
  const int first_m = group * kGroupM;
  const int gsize = (ntm - first_m) < kGroupM ? (ntm - first_m) : kGroupM;
  const int inner = bp - group * per_group;
  tm = first_m + inner % gsize;
  tn = inner / gsize;
}

template <int BM, int BN, int KIND, int YDT>
__global__ __launch_bounds__(kThreads, 1) void k_gemm(const GemmArgs g) {
  using MM = typename std::conditional<KIND == GEMM_FP8, MmaF8, MmaI8>::type;
  using TL = Tile<BM, BN>;
  using Acc = typename MM::Acc;
  constexpr int NR = MM::NR;
  constexpr int KS = kBK / MM::KSTEP;

  // the LDS buffers as distinct objects, so the compiler can tell the buffers
  // the DMA is filling from the one the fragment reads come from
  __shared__ __attribute__((aligned(16))) uint8_t sa0[BM * kBK], sb0[BN * kBK];
  __shared__ __attribute__((aligned(16))) uint8_t sa1[BM * kBK], sb1[BN * kBK];
  __shared__ __attribute__((aligned(16))) uint8_t sa2[BM * kBK], sb2[BN * kBK];
  __shared__ __attribute__((aligned(16))) uint8_t sa3[BM * kBK], sb3[BN * kBK];

  const int M = (int)g.M, N = (int)g.N, K = (int)g.K;
  const int ntm = (M + BM - 1) / BM, ntn = (N + BN - 1) / BN;
  int tm, tn;
  tile_coords(ntm, ntn, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- DMA loader.  One wave instruction fills 1 KB = 16 LDS rows; lane l
  // lands at row l/4, physical chunk l%4, which holds logical chunk
  // (l%4) ^ ((row >> 1) & 3).  Rows past M (or N) re-read the last row: they
  // only feed outputs that are never stored.
  constexpr int kRowsPerDma = 64 * 16 / kBK;     // 16
  const int lrow = lane >> 2;
  const int lchunk = (lane & 3) ^ ((lrow >> 1) & 3);
  uint32_t aoff[TL::ALOADS], boff[TL::BLOADS];
#pragma unroll
  for (int j = 0; j < TL::ALOADS; ++j) {
    int gm = m0 + (j * (kThreads / 64) + wave) * kRowsPerDma + lrow;
    gm = gm < M ? gm : M - 1;
    aoff[j] = (uint32_t)(gm * K + lchunk * 16);
  }
#pragma unroll
  for (int j = 0; j < TL::BLOADS; ++j) {
    int gn = n0 + (j * (kThreads / 64) + wave) * kRowsPerDma + lrow;
    gn = gn < N ? gn : N - 1;
    boff[j] = (uint32_t)(gn * K + lchunk * 16);
  }
  auto dma = [&](uint8_t* sa, uint8_t* sb, int k0) {
    const uint8_t* abase = g.a + k0;
    const uint8_t* bbase = g.b + k0;
#pragma unroll
    for (int j = 0; j < TL::ALOADS; ++j)
      __builtin_amdgcn_global_load_lds((gptr_t)(abase + aoff[j]),
                                       (lptr_t)(sa + (j * (kThreads / 64) + wave) * kRowsPerDma * kBK), 16,
                                       0, 0);
#pragma unroll
    for (int j = 0; j < TL::BLOADS; ++j)
      __builtin_amdgcn_global_load_lds((gptr_t)(bbase + boff[j]),
                                       (lptr_t)(sb + (j * (kThreads / 64) + wave) * kRowsPerDma * kBK), 16,
                                       0, 0);
  };
  // Register loader for a last stage that K does not fill: chunks past K are
  // zero so they add nothing to the dot products.
  auto tail = [&](uint8_t* sa, uint8_t* sb, int k0) {
#pragma unroll
    for (int j = 0; j < TL::ALOADS; ++j) {
      const int i = tid + j * kThreads, row = i >> 2, c = i & 3;
      const int gm = (m0 + row) < M ? (m0 + row) : M - 1;
      const int gk = k0 + c * 16;
      *(v4i*)(sa + swz(row, c)) = gk < K ? *(const v4i*)(g.a + gm * K + gk) : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < TL::BLOADS; ++j) {
      const int i = tid + j * kThreads, row = i >> 2, c = i & 3;
      const int gn = (n0 + row) < N ? (n0 + row) : N - 1;
      const int gk = k0 + c * 16;
      *(v4i*)(sb + swz(row, c)) = gk < K ? *(const v4i*)(g.b + gn * K + gk) : v4i{0, 0, 0, 0};
    }
  };
  const int nfull = K / kBK;                 // stages filled by DMA
  const bool ragged = (K % kBK) != 0;        // one more, partial stage at the end

  Acc acc[TL::FM][TL::FN];
#pragma unroll
  for (int i = 0; i < TL::FM; ++i)
#pragma unroll
    for (int j = 0; j < TL::FN; ++j) acc[i][j] = Acc{};

  // Byte offset of this lane's operand row in the A / B stage, and of its
  // chunk inside the row.
  const int arow = (wm * TL::TM + (lane & 31)) * kBK;
  const int brow = (wn * TL::TN + (lane & 31)) * kBK;
  const int loff = MM::lane_off(lane);
  // B fragments are double buffered across k-steps; each A fragment is
  // re-read for the next k-step right after its last MFMA of this one.
  auto compute = [&](const uint8_t* As, const uint8_t* Bs) {
    const uint8_t* ar = As + arow;
    const uint8_t* br = Bs + brow;
    typename MM::Op af[TL::FM], bf[2][TL::FN];
#pragma unroll
    for (int i = 0; i < TL::FM; ++i) af[i] = MM::load(ar + i * 32 * kBK, loff, 0);
#pragma unroll
    for (int j = 0; j < TL::FN; ++j) bf[0][j] = MM::load(br + j * 32 * kBK, loff, 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < KS) {
#pragma unroll
        for (int j = 0; j < TL::FN; ++j) bf[cur ^ 1][j] = MM::load(br + j * 32 * kBK, loff, ks + 1);
      }
#pragma unroll
      for (int i = 0; i < TL::FM; ++i) {
#pragma unroll
        for (int j = 0; j < TL::FN; ++j) acc[i][j] = MM::mma(af[i], bf[cur][j], acc[i][j]);
        if (ks + 1 < KS) af[i] = MM::load(ar + i * 32 * kBK, loff, ks + 1);
      }
    }
  };
  // ---- main loop.  Stage s lives in buffer s % 4 and is requested three
  // stages ahead.  Before computing stage s a wave waits until at most the
  // DMA of stages s+1, s+2 is outstanding (its own loads retire in order),
  // then the barrier makes every wave's copy of stage s visible and proves
  // that stage s-1's buffer, refilled next with stage s+3, has been read.
  auto wait_stage = [&](int s) {
    const int later = (nfull - 1 - s) < 2 ? (nfull - 1 - s) : 2;   // stages issued after s
    if (later >= 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * TL::LOADS) : "memory");
    else if (later == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(TL::LOADS) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  auto stage = [&](int s, const uint8_t* ca, const uint8_t* cb, uint8_t* na, uint8_t* nb) {
    wait_stage(s);
    if (s + 3 < nfull) dma(na, nb, (s + 3) * kBK);
    compute(ca, cb);
  };
  if (nfull > 0) dma(sa0, sb0, 0);
  if (nfull > 1) dma(sa1, sb1, kBK);
  if (nfull > 2) dma(sa2, sb2, 2 * kBK);
  int kt = 0;
  for (; kt + 4 <= nfull; kt += 4) {          // single exit: the accumulators stay in place
    stage(kt, sa0, sb0, sa3, sb3);
    stage(kt + 1, sa1, sb1, sa0, sb0);
    stage(kt + 2, sa2, sb2, sa1, sb1);
    stage(kt + 3, sa3, sb3, sa2, sb2);
  }
  if (kt < nfull) stage(kt, sa0, sb0, sa3, sb3);
  if (kt + 1 < nfull) stage(kt + 1, sa1, sb1, sa0, sb0);
  if (kt + 2 < nfull) stage(kt + 2, sa2, sb2, sa1, sb1);
  // ---- the partial last stage, through registers, in buffer nfull % 4 (last
  // read by stage nfull - 4, long finished)
  if (ragged) {
    const int b = nfull & 3;
    uint8_t* ta = b == 0 ? sa0 : b == 1 ? sa1 : b == 2 ? sa2 : sa3;
    uint8_t* tb = b == 0 ? sb0 : b == 1 ? sb1 : b == 2 ? sb2 : sb3;
    __syncthreads();                          // every wave is past stage nfull - 4
    tail(ta, tb, nfull * kBK);
    __syncthreads();
    compute(ta, tb);
  }

  // ---- epilogue.  Register r of fragment (i, j) is output
  // (mw + i*32 + out_row(r), nw + j*32 + lane%32).  Row factors are loaded
  // once per fragment row, column factors once per fragment.
  const int mw = m0 + wm * TL::TM, nw = n0 + wn * TL::TN;
  const int ocol = lane & 31;
  const bool full = (m0 + BM <= M) && (n0 + BN <= N);
  if constexpr (KIND == GEMM_FP8 || KIND == GEMM_INT8) {
#pragma unroll
    for (int i = 0; i < TL::FM; ++i) {
      float sx[NR];
      int rs[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const int m = mw + i * 32 + out_row(r, lane);
        const int mc = m < M ? m : M - 1;
        sx[r] = g.a_scale[mc];
        if constexpr (KIND == GEMM_INT8) rs[r] = g.a_rowsum[mc];
      }
#pragma unroll
      for (int j = 0; j < TL::FN; ++j) {
        const int n = nw + j * 32 + ocol;
        const int nc = n < N ? n : N - 1;
        const float sb = g.b_scale[nc];
        const float bb = g.bias ? g.bias[nc] : 0.0f;
        int zb = 0;
        if constexpr (KIND == GEMM_INT8) zb = (int)g.b_zp[nc];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const int m = mw + i * 32 + out_row(r, lane);
          if (!full && (m >= M || n >= N)) continue;
          const int o = m * N + n;
          float v;
          if constexpr (KIND == GEMM_INT8) {
            const int a = acc[i][j][r];
            if (g.acc_out) g.acc_out[o] = a;
            v = (sx[r] * sb) * (float)(a - zb * rs[r]) + bb;
          } else {
            v = acc[i][j][r] * (sx[r] * sb) + bb;
          }
          store_out<YDT>(g.y, o, v);
        }
      }
    }
  } else {
    // LLM.int8: dequantize the int8 part in place (the fp32 value replaces
    // the int32 in the same registers), then add the outlier flow with
    // v_mfma_f32_32x32x16_f16 whose accumulator input is that value (its
    // output layout is the same 32 x 32 layout).
#pragma unroll
    for (int i = 0; i < TL::FM; ++i) {
#pragma unroll
      for (int j = 0; j < TL::FN; ++j) {
        const int n = nw + j * 32 + ocol;
        const int nc = n < N ? n : N - 1;
        const float sb = g.b_scale[nc];
        const int zb = (int)g.b_zp[nc];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const int m = mw + i * 32 + out_row(r, lane);
          const int mc = m < M ? m : M - 1;
          const int a = acc[i][j][r];
          if (g.acc_out && m < M && n < N) g.acc_out[m * N + n] = a;
          acc[i][j][r] = __float_as_int((g.a_scale[mc] * sb) * (float)(a - zb * g.a_rowsum[mc]));
        }
      }
    }
    const int cnt = *g.out_cnt;
    const int kg = lane >> 5;                          // 8-column group of the 16-column step
    const int orow = lane & 31;
    for (int kc = 0; kc < cnt; kc += 16) {
      int col[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int jj = kc + kg * 8 + e;
        col[e] = jj < cnt ? g.out_idx[jj] : -1;
      }
      v8h xo[TL::FM], wo[TL::FN];
#pragma unroll
      for (int i = 0; i < TL::FM; ++i) {
        const int m = mw + i * 32 + orow;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          xo[i][e] = (col[e] >= 0 && m < M) ? __builtin_bit_cast(_Float16, g.x_f16[m * K + col[e]])
                                            : (_Float16)0.0f;
      }
#pragma unroll
      for (int j = 0; j < TL::FN; ++j) {
        const int n = nw + j * 32 + orow;
        const bool nok = n < N;
        const float sb = nok ? g.b_scale[n] : 0.0f;
        const float zb = nok ? g.b_zp[n] : 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float wv = 0.0f;
          if (col[e] >= 0 && nok) wv = sb * ((float)(int8_t)g.b[n * K + col[e]] - zb);
          wo[j][e] = (_Float16)wv;
        }
      }
#pragma unroll
      for (int i = 0; i < TL::FM; ++i)
#pragma unroll
        for (int j = 0; j < TL::FN; ++j) {
          v16f c = __builtin_bit_cast(v16f, acc[i][j]);
          c = __builtin_amdgcn_mfma_f32_32x32x16_f16(xo[i], wo[j], c, 0, 0, 0);
          acc[i][j] = __builtin_bit_cast(v16i, c);
        }
    }
#pragma unroll
    for (int j = 0; j < TL::FN; ++j) {
      const int n = nw + j * 32 + ocol;
      if (n >= N) continue;
      const float bb = g.bias ? g.bias[n] : 0.0f;
#pragma unroll
      for (int i = 0; i < TL::FM; ++i)
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const int m = mw + i * 32 + out_row(r, lane);
          if (m < M) store_out<YDT>(g.y, m * N + n, __int_as_float(acc[i][j][r]) + bb);
        }
    }
  }
}

template <int BM, int BN, int KIND>
hipError_t launch_tiles(const GemmArgs& g, int ydt, hipStream_t st) {
  const int64_t ntm = (g.M + BM - 1) / BM, ntn = (g.N + BN - 1) / BN;
  dim3 grid((unsigned)(ntm * ntn)), block(kThreads);
  switch (ydt) {
    case DT_F32: k_gemm<BM, BN, KIND, DT_F32><<<grid, block, 0, st>>>(g); break;
    case DT_F16: k_gemm<BM, BN, KIND, DT_F16><<<grid, block, 0, st>>>(g); break;
    default: k_gemm<BM, BN, KIND, DT_BF16><<<grid, block, 0, st>>>(g); break;
  }
  return hipGetLastError();
}

// Pick the largest tile that still gives most of the 256 CUs a workgroup.
template <int KIND>
hipError_t launch_kind(const GemmArgs& g, int ydt, hipStream_t st) {
  auto tiles = [&](int bm, int bn) { return ((g.M + bm - 1) / bm) * ((g.N + bn - 1) / bn); };
  // the outlier flow needs the accumulators in VGPRs: no 256 x 256 tile there
  if constexpr (KIND != GEMM_INT8_DECOMP) {
    if (tiles(256, 256) >= 192) return launch_tiles<256, 256, KIND>(g, ydt, st);
  }
  if (tiles(128, 128) >= 192) return launch_tiles<128, 128, KIND>(g, ydt, st);
  return launch_tiles<64, 64, KIND>(g, ydt, st);
}

}  // namespace

hipError_t launch_gemm(GemmKind kind, const GemmArgs& g, int ydt, hipStream_t st) {
  switch (kind) {
    case GEMM_INT8: return launch_kind<GEMM_INT8>(g, ydt, st);
    case GEMM_INT8_DECOMP: return launch_kind<GEMM_INT8_DECOMP>(g, ydt, st);
    default: return launch_kind<GEMM_FP8>(g, ydt, st);
  }
}

}  // namespace q8
