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
//   GEMM_FP8          v_mfma_f32_16x16x128_f8f6f4 on e4m3 codes, fp32
//                     accumulation, y = S_a[m] S_b[n] acc (+ bias)
//
// Tiling: a workgroup of 4 waves (2 x 2) owns a BM x BN output tile; each wave
// owns (BM/2) x (BN/2) built from MFMA fragments (32 x 32 int8, 16 x 16 fp8).  K advances 128 bytes per
// stage.  Stages are double buffered in LDS: while the MFMAs consume stage k,
// the next stage's global loads are in flight in registers.  The 16-byte
// chunks of each 128-byte LDS row are XOR-swizzled by (row & 7), so the
// fragment reads (rows 0..7 of one chunk column in one LDS cycle) hit 8
// distinct bank groups.  Workgroups are renumbered so that consecutive tiles
// land on the same XCD (the dispatcher deals workgroups round-robin over the 8
// XCDs) and, within an XCD, 4 tile-rows share each weight tile in L2.
#include "q8_device.hpp"
#include "q8_kernels.hpp"

namespace q8 {
namespace {

constexpr int kBK = 128;            // bytes of K per stage
constexpr int kThreads = 256;       // 4 waves
constexpr int kGroupM = 4;          // tile-rows per L2 group
constexpr int kXcds = 8;

__device__ __forceinline__ int swz(int row, int chunk) { return row * kBK + ((chunk ^ (row & 7)) << 4); }

// One MFMA shape: operand fragment loads from the swizzled LDS stage, the
// instruction, and where output register r of a lane lands in the fragment.
// A and B fragments use the same lane -> k mapping, so each instruction sums
// over exactly the k bytes of its step whatever order the hardware uses.
struct MmaI8 {                       // v_mfma_i32_32x32x32_i8
  static constexpr int F = 32, KSTEP = 32, NR = 16;
  using Op = v4i;
  using Acc = v16i;
  // lane l: row l % 32, 16-byte chunk l / 32 of the 32-byte k-step
  __device__ static Op load(const uint8_t* S, int row, int ks, int lane) {
    return *(const v4i*)(S + swz(row, ks * 2 + (lane >> 5)));
  }
  __device__ static Acc mma(const Op& a, const Op& b, const Acc& c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
  }
  __device__ static int op_row(int lane) { return lane & 31; }
  __device__ static int out_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }
  __device__ static int out_col(int lane) { return lane & 31; }
};
struct MmaF8 {                       // v_mfma_f32_16x16x128_f8f6f4, both operands e4m3
  static constexpr int F = 16, KSTEP = 128, NR = 4;
  using Op = v8i;
  using Acc = v4f;
  // lane l: row l % 16, 32-byte chunk l / 16 of the 128-byte k-step
  __device__ static Op load(const uint8_t* S, int row, int ks, int lane) {
    const int c = 2 * (lane >> 4);
    const v4i lo = *(const v4i*)(S + swz(row, c));
    const v4i hi = *(const v4i*)(S + swz(row, c + 1));
    return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  __device__ static Acc mma(const Op& a, const Op& b, const Acc& c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
  }
  __device__ static int op_row(int lane) { return lane & 15; }
  __device__ static int out_row(int r, int lane) { return 4 * (lane >> 4) + r; }
  __device__ static int out_col(int lane) { return lane & 15; }
};

template <int BM, int BN, class MM>
struct Tile {
  static constexpr int TM = BM / 2, TN = BN / 2;            // wave tile
  static constexpr int FM = TM / MM::F, FN = TN / MM::F;    // fragments per wave
  static constexpr int ALOADS = BM * (kBK / 16) / kThreads;
  static constexpr int BLOADS = BN * (kBK / 16) / kThreads;
  static constexpr int STAGE = (BM + BN) * kBK;             // bytes per LDS stage
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
  using TL = Tile<BM, BN, MM>;
  using Acc = typename MM::Acc;
  constexpr int NR = MM::NR;

  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * TL::STAGE];

  const int64_t M = g.M, N = g.N, K = g.K;
  const int ntm = (int)((M + BM - 1) / BM), ntn = (int)((N + BN - 1) / BN);
  int tm, tn;
  tile_coords(ntm, ntn, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- global -> register -> LDS loader (16 bytes per thread per load)
  v4i ra[TL::ALOADS], rb[TL::BLOADS];
  auto gload = [&](int kt) {
    const int64_t k0 = (int64_t)kt * kBK;
#pragma unroll
    for (int j = 0; j < TL::ALOADS; ++j) {
      const int i = tid + j * kThreads, row = i >> 3, c = i & 7;
      const int64_t gm = m0 + row, gk = k0 + c * 16;
      ra[j] = (gm < M && gk < K) ? *(const v4i*)(g.a + gm * K + gk) : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < TL::BLOADS; ++j) {
      const int i = tid + j * kThreads, row = i >> 3, c = i & 7;
      const int64_t gn = n0 + row, gk = k0 + c * 16;
      rb[j] = (gn < N && gk < K) ? *(const v4i*)(g.b + gn * K + gk) : v4i{0, 0, 0, 0};
    }
  };
  auto sstore = [&](int buf) {
    uint8_t* As = smem + buf * TL::STAGE;
    uint8_t* Bs = As + BM * kBK;
#pragma unroll
    for (int j = 0; j < TL::ALOADS; ++j) {
      const int i = tid + j * kThreads;
      *(v4i*)(As + swz(i >> 3, i & 7)) = ra[j];
    }
#pragma unroll
    for (int j = 0; j < TL::BLOADS; ++j) {
      const int i = tid + j * kThreads;
      *(v4i*)(Bs + swz(i >> 3, i & 7)) = rb[j];
    }
  };

  Acc acc[TL::FM][TL::FN];
#pragma unroll
  for (int i = 0; i < TL::FM; ++i)
#pragma unroll
    for (int j = 0; j < TL::FN; ++j) acc[i][j] = Acc{};

  const int orow = MM::op_row(lane);
  auto compute = [&](int buf) {
    const uint8_t* As = smem + buf * TL::STAGE;
    const uint8_t* Bs = As + BM * kBK;
#pragma unroll
    for (int ks = 0; ks < kBK / MM::KSTEP; ++ks) {
      typename MM::Op af[TL::FM], bf[TL::FN];
#pragma unroll
      for (int i = 0; i < TL::FM; ++i) af[i] = MM::load(As, wm * TL::TM + i * MM::F + orow, ks, lane);
#pragma unroll
      for (int j = 0; j < TL::FN; ++j) bf[j] = MM::load(Bs, wn * TL::TN + j * MM::F + orow, ks, lane);
#pragma unroll
      for (int i = 0; i < TL::FM; ++i)
#pragma unroll
        for (int j = 0; j < TL::FN; ++j) acc[i][j] = MM::mma(af[i], bf[j], acc[i][j]);
    }
  };

  // ---- main loop: one barrier per stage
  const int nk = (int)((K + kBK - 1) / kBK);
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) gload(kt + 1);
    compute(kt & 1);
    if (more) sstore((kt + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: register r of fragment (i, j) is output
  // (mw + i*F + out_row(r), nw + j*F + out_col)
  const int64_t mw = m0 + wm * TL::TM, nw = n0 + wn * TL::TN;
  const int ocol = MM::out_col(lane);
  if constexpr (KIND == GEMM_FP8) {
#pragma unroll
    for (int j = 0; j < TL::FN; ++j) {
      const int64_t n = nw + j * MM::F + ocol;
      if (n >= N) continue;
      const float sb = g.b_scale[n];
      const float bb = g.bias ? g.bias[n] : 0.0f;
#pragma unroll
      for (int i = 0; i < TL::FM; ++i)
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const int64_t m = mw + i * MM::F + MM::out_row(r, lane);
          if (m < M) store_out<YDT>(g.y, m * N + n, acc[i][j][r] * (g.a_scale[m] * sb) + bb);
        }
    }
  } else if constexpr (KIND == GEMM_INT8) {
    // zero-point correction in int32, then fp32 scaling, stored at once
#pragma unroll
    for (int j = 0; j < TL::FN; ++j) {
      const int64_t n = nw + j * MM::F + ocol;
      if (n >= N) continue;
      const float sb = g.b_scale[n];
      const int zb = (int)g.b_zp[n];
      const float bb = g.bias ? g.bias[n] : 0.0f;
#pragma unroll
      for (int i = 0; i < TL::FM; ++i)
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const int64_t m = mw + i * MM::F + MM::out_row(r, lane);
          if (m < M) {
            const int a = acc[i][j][r];
            if (g.acc_out) g.acc_out[m * N + n] = a;
            const int c = a - zb * g.a_rowsum[m];
            store_out<YDT>(g.y, m * N + n, (g.a_scale[m] * sb) * (float)c + bb);
          }
        }
    }
  } else {
    // LLM.int8: dequantize the int8 part in place (the fp32 value replaces
    // the int32 in the same registers), then add the outlier flow with
    // v_mfma_f32_32x32x16_f16 whose accumulator input is that value.  Its
    // output layout is the 32 x 32 layout of the int8 instruction.
#pragma unroll
    for (int j = 0; j < TL::FN; ++j) {
      const int64_t n = nw + j * MM::F + ocol;
      const bool nok = n < N;
      const float sb = nok ? g.b_scale[n] : 0.0f;
      const int zb = nok ? (int)g.b_zp[n] : 0;
#pragma unroll
      for (int i = 0; i < TL::FM; ++i)
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const int64_t m = mw + i * MM::F + MM::out_row(r, lane);
          const bool ok = nok && m < M;
          const int a = acc[i][j][r];
          if (ok && g.acc_out) g.acc_out[m * N + n] = a;
          const int c = a - zb * (ok ? g.a_rowsum[m] : 0);
          acc[i][j][r] = __float_as_int((ok ? g.a_scale[m] * sb : 0.0f) * (float)c);
        }
    }
    const int cnt = *g.out_cnt;
    const int kg = lane >> 5;                          // 8-column group of the 16-column step
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
        const int64_t m = mw + i * MM::F + orow;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          xo[i][e] = (col[e] >= 0 && m < M) ? __builtin_bit_cast(_Float16, g.x_f16[m * K + col[e]])
                                            : (_Float16)0.0f;
      }
#pragma unroll
      for (int j = 0; j < TL::FN; ++j) {
        const int64_t n = nw + j * MM::F + orow;
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
      const int64_t n = nw + j * MM::F + ocol;
      if (n >= N) continue;
      const float bb = g.bias ? g.bias[n] : 0.0f;
#pragma unroll
      for (int i = 0; i < TL::FM; ++i)
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const int64_t m = mw + i * MM::F + MM::out_row(r, lane);
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
