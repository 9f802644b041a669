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
// owns (BM/2) x (BN/2) built from 32 x 32 MFMA fragments.  The int8 tiles of
// 256 x 256, 128 x 128 and 64 x 128 use 8 waves (2 x 4, two per SIMD), each
// (BM/2) x (BN/4).  K advances 64 bytes per stage on 256 x 256 tiles, 128 on
// the smaller ones.  Four LDS buffers hold four stages, filled by
// global_load_lds_dwordx4 (global -> LDS without registers) three stages
// ahead of the MFMAs, so a stage's loads have three stages of compute to
// arrive.  Fragments are double buffered in registers: the LDS reads of the
// next k-step (across a stage boundary: of the next stage, right after its
// barrier) are issued before the MFMAs of the current one.
//
// LDS layout: row-major 64-byte rows (one row of the tile, one stage of K),
// the 16-byte chunk c of row r stored at chunk position c ^ ((r >> 2) & 3).
// gfx950's LDS serves a ds_read_b128 16 lanes per cycle over 64 four-byte
// banks (256 bytes), i.e. four 64-byte rows: a fragment read has rows 0..15
// of one logical chunk in one cycle, rows r, r+4, r+8, r+12 share a bank
// quarter, and the XOR gives those four rows four different 16-byte slots of
// it.  (The bank-conflict counter reads half of all LDS cycles with the
// 32-bank pattern c ^ ((r >> 1) & 3), and none with this one.)  The DMA writes 64
// consecutive 16-byte slots per wave instruction, so the swizzle is applied
// on the global side: each lane fetches the chunk that belongs at its slot.
//
// Workgroups are renumbered so consecutive tiles land on the same XCD (the
// dispatcher deals workgroups round-robin over the 8 XCDs) and, within an
// XCD, 4 tile-rows share each weight tile in L2.
//
// Indices are 32-bit: the host guarantees M*K, N*K and M*N are below 2^31.
#include <climits>

#include "q8_device.hpp"
#include "q8_kernels.hpp"

namespace q8 {
static_assert(DT_I8 == kOutInt8, "INT8 output code");
namespace {


// Bytes of K per stage: 64 for the 256 x 256 tile (four stages of 32 KB),
// kSmallBK for the smaller tiles, whose four stages fit at 128 bytes
// (whole 128-byte lines per DMA lane group)
constexpr int kSmallBK = 128;
constexpr int bk_for(int bm) { return bm == 256 ? 64 : kSmallBK; }
constexpr int kStages = 4;          // LDS buffers (prefetch distance kStages - 1)
constexpr int kGroupM = 4;          // tile-rows per L2 group
constexpr int kXcds = 8;
constexpr int kMaxGroupsDev = 1024;   // groups (experts) of one grouped call

// LDS row swizzle: 16-byte chunk c of row r sits at physical chunk
// c ^ sw(r).  With 64-byte rows four rows share a 256-byte bank row, with
// 128-byte rows two; either way the 16 rows that one 16-lane group of a
// fragment read touches cover all 64 banks once.
template <int BK>
__device__ __forceinline__ int swz_key(int row) { return BK == 64 ? (row >> 2) & 3 : (row >> 1) & 7; }
template <int BK>
__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ swz_key<BK>(row)) << 4); }

// One MFMA shape.  A fragment row is (base multiple of 32) + lane % 32, so
// swz_key(row) == swz_key(lane % 32) and the swizzled byte offset of the
// lane's operand inside its LDS row is lane_off(lane) XOR a per-k-step constant.
// A and B fragments use the same lane -> k mapping, so each instruction sums
// over exactly the k bytes of its step whatever order the hardware uses.
struct MmaI8 {                       // v_mfma_i32_32x32x32_i8
  static constexpr int KSTEP = 32, NR = 16;
  using Op = v4i;
  using Acc = v16i;
  // lane l: 16-byte logical chunk 2*ks + l/32 of its row
  template <int BK>
  __device__ static int lane_off(int lane) { return ((lane >> 5) ^ swz_key<BK>(lane & 31)) << 4; }
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
  template <int BK>
  __device__ static int lane_off(int lane) { return ((2 * (lane >> 5)) ^ swz_key<BK>(lane & 31)) << 4; }
  __device__ static Op load(const uint8_t* row, int off, int ks) {
    const v4i lo = *(const v4i*)(row + (off ^ (ks << 6)));
    const v4i hi = *(const v4i*)(row + ((off ^ 16) ^ (ks << 6)));
    return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  __device__ static Acc mma(const Op& a, const Op& b, const Acc& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
  }
};
// The 32-bit pattern of an accumulator element, taken by value: a bit_cast
// applied directly to an element of an ext_vector_type is lowered to a read
// of element 0 by this compiler.
__device__ __forceinline__ int raw32(int x) { return x; }
__device__ __forceinline__ int raw32(float x) { return __float_as_int(x); }

// 32 x 32 output fragment layout (all 32x32 MFMAs): register r of lane l is
// row 8*(r/4) + 4*(l/32) + r%4, column l%32.
__device__ __forceinline__ int out_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

template <int BM, int BN, int NW, int BK>
struct Tile {
  static constexpr int NT = 64 * NW;                        // threads
  static constexpr int WN = NW == 8 ? 4 : 2, WM = NW / WN;  // wave grid
  static constexpr int TM = BM / WM, TN = BN / WN;          // wave tile
  static constexpr int FM = TM / 32, FN = TN / 32;          // 32x32 fragments per wave
  static constexpr int ALOADS = BM * (BK / 16) / NT;   // 16-byte chunks per thread
  static constexpr int BLOADS = BN * (BK / 16) / NT;
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

// Grouped problems (experts over routed rows): rows offsets[e] .. offsets[e+1]-1
// of A and Y belong to group e, whose B and column scales start at e N K and
// e N.  Tile t of the launch is tile-column t % ntn of tile-row t / ntn,
// counted over the groups' tile-rows in order; the offsets are clamped to
// [0, M] and made non-decreasing, so no group reaches outside the arrays.
// Returns false for the tiles past the last group (the grid is an upper bound).
//
// The workgroup resolves its tile in parallel: the clamped offsets are the
// running maximum of max(offsets[e], 0) capped at M (group e spans c[e] ..
// c[e+1]), and the groups' tile-row counts are summed by a block scan, so a
// workgroup reads the E + 1 offsets once, split over its threads, and finds
// its group by binary search: O(E / threads + log E) per workgroup.
template <int NT>
__device__ __forceinline__ int block_scan_incl(int v, int* red, bool max_op) {
  const int t = threadIdx.x;
  red[t] = v;
  __syncthreads();
#pragma unroll
  for (int d = 1; d < NT; d <<= 1) {
    const int o = t >= d ? red[t - d] : (max_op ? INT_MIN : 0);
    __syncthreads();
    v = max_op ? (v > o ? v : o) : v + o;
    red[t] = v;
    __syncthreads();
  }
  return v;
}

template <int BM, int BN, int ES, int NT>
__device__ __forceinline__ bool group_tile(GemmArgs& g, int& tm, int& tn, int* lds) {
  const int T = (int)g.M, N = (int)g.N, K = (int)g.K, E = g.groups;
  const int ntn = (N + BN - 1) / BN;
  const int t = blockIdx.x, tid = threadIdx.x;
  tn = t % ntn;
  const int r = t / ntn;
  int* const c = lds;                 // [E + 1] clamped offsets
  int* const R = lds + (E + 1);       // [E + 1] first tile-row of each group
  int* const red = R + (E + 1);       // [NT] scan scratch
  const int per = (E + 1 + NT - 1) / NT, lo = tid * per;
  const int hi = lo + per < E + 1 ? lo + per : E + 1;
  // running maximum of max(offsets, 0) over this thread's slice, then across threads
  int m = 0;
  for (int e = lo; e < hi; ++e) m = g.group_offsets[e] > m ? g.group_offsets[e] : m;
  const int incl = block_scan_incl<NT>(m, red, true);
  int run = tid > 0 ? red[tid - 1] : 0;       // exclusive: the maximum before this slice
  run = run > 0 ? run : 0;
  for (int e = lo; e < hi; ++e) {
    run = g.group_offsets[e] > run ? g.group_offsets[e] : run;
    c[e] = run < T ? run : T;
  }
  (void)incl;
  __syncthreads();
  // tile-rows of the groups in this slice, then their running sum
  int cnt = 0;
  for (int e = lo; e < hi && e < E; ++e) cnt += (c[e + 1] - c[e] + BM - 1) / BM;
  block_scan_incl<NT>(cnt, red, false);
  int acc = tid > 0 ? red[tid - 1] : 0;
  for (int e = lo; e < hi; ++e) {
    R[e] = acc;
    if (e < E) acc += (c[e + 1] - c[e] + BM - 1) / BM;
  }
  __syncthreads();
  const bool inside = r < R[E];
  int e = 0;
  if (inside) {                       // the last group whose first tile-row is <= r
    int lo2 = 0, hi2 = E - 1;
    while (lo2 < hi2) {
      const int mid = (lo2 + hi2 + 1) >> 1;
      if (R[mid] <= r) lo2 = mid;
      else hi2 = mid - 1;
    }
    e = lo2;
  }
  // every lane holds the same values: make them scalar for the DMA bases
  const int a = __builtin_amdgcn_readfirstlane(c[e]), b = __builtin_amdgcn_readfirstlane(c[e + 1]);
  const int trow = __builtin_amdgcn_readfirstlane(r - R[e]);
  e = __builtin_amdgcn_readfirstlane(e);
  const bool in = __builtin_amdgcn_readfirstlane(inside ? 1 : 0) != 0;
  __syncthreads();                    // the LDS is the main loop's next
  if (!in) return false;
  tm = trow;
  g.M = b - a;
  g.a += (size_t)a * K;
  g.a_scale += a;
  g.y = (uint8_t*)g.y + (size_t)a * N * ES;
  g.b += (size_t)e * N * K;
  g.b_scale += (size_t)e * N;
  return true;
}

template <int BM, int BN, int KIND, int YDT, int NW, bool GROUPED = false>
__global__ __launch_bounds__(64 * NW, 1) void k_gemm(const GemmArgs g0) {
  using MM = typename std::conditional<KIND == GEMM_FP8, MmaF8, MmaI8>::type;
  constexpr int kBK = bk_for(BM);
  using TL = Tile<BM, BN, NW, kBK>;
  constexpr int kThreads = TL::NT;
  using Acc = typename MM::Acc;
  constexpr int NR = MM::NR;
  constexpr int KS = kBK / MM::KSTEP;

  // one LDS arena: four stages of A and B tiles in the main loop, then the
  // epilogue's factor arrays and output staging
  constexpr int kStageBytes = (BM + BN) * kBK;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kStages * kStageBytes];
  uint8_t* const sa0 = smem;
  uint8_t* const sb0 = smem + BM * kBK;
  uint8_t* const sa1 = smem + kStageBytes;
  uint8_t* const sb1 = sa1 + BM * kBK;
  uint8_t* const sa2 = smem + 2 * kStageBytes;
  uint8_t* const sb2 = sa2 + BM * kBK;
  uint8_t* const sa3 = smem + 3 * kStageBytes;
  uint8_t* const sb3 = sa3 + BM * kBK;

  GemmArgs g = g0;
  int tm, tn;
  if constexpr (GROUPED) {
    static_assert(2 * (kMaxGroupsDev + 1) * 4 + kThreads * 4 <= kStages * kStageBytes, "group scan does not fit");
    if (!group_tile<BM, BN, YDT == DT_F32 ? 4 : 2, kThreads>(g, tm, tn, (int*)smem)) return;   // uniform
  } else {
    tile_coords((int)((g.M + BM - 1) / BM), (int)((g.N + BN - 1) / BN), tm, tn);
  }
  const int M = (int)g.M, N = (int)g.N, K = (int)g.K;
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / TL::WN, wn = wave % TL::WN;

  // Epilogue factors, loaded now and parked in registers (thread t: row m0+t
  // and column n0+t of the tile), so their latency is long over when the
  // epilogue puts them in LDS.
  float pf_sx = 0.0f, pf_sb = 0.0f, pf_bb = 0.0f;
  int pf_rs = 0, pf_zi = 0;
  if (tid < BM) {
    const int m = m0 + tid < M ? m0 + tid : M - 1;
    pf_sx = g.a_scale[m];
    if constexpr (KIND != GEMM_FP8) pf_rs = g.a_rowsum[m];
  }
  if (tid < BN) {
    const int n = n0 + tid < N ? n0 + tid : N - 1;
    pf_sb = g.b_scale[n];
    if constexpr (KIND != GEMM_FP8) pf_zi = (int)g.b_zp[n];
    pf_bb = g.bias ? g.bias[n] : 0.0f;
  }
  // LLM.int8: the outlier count and this lane's 16 bytes of the panels of
  // the first kPanelCols outlier columns (fragment rows m and n, 8-column
  // group lane / 32), requested now so that the epilogue's outlier flow does
  // not begin with a round trip.  Rows past M or N read the last row; their
  // outputs are not stored.
  int pf_cnt = 0;
  v4i pf_xo[TL::FM], pf_wo[TL::FN];
  if constexpr (KIND == GEMM_INT8_DECOMP) {
    pf_cnt = *g.out_cnt;
    const int kg0 = lane >> 5, lm0 = lane & 31;
#pragma unroll
    for (int i = 0; i < TL::FM; ++i) {
      const int m = m0 + wm * TL::TM + i * 32 + lm0;
      const int mc = m < M ? m : M - 1;
      pf_xo[i] = *(const v4i*)(g.x_panel + (size_t)mc * kPanelCols + kg0 * 8);
    }
#pragma unroll
    for (int j = 0; j < TL::FN; ++j) {
      const int n = n0 + wn * TL::TN + j * 32 + lm0;
      const int ncl = n < N ? n : N - 1;
      pf_wo[j] = *(const v4i*)(g.w_panel + (size_t)ncl * kPanelCols + kg0 * 8);
    }
  }

  // ---- DMA loader.  One wave instruction fills 1 KB = 1024 / kBK LDS rows;
  // lane l lands at row l / (kBK/16) of them, physical chunk l % (kBK/16),
  // which holds logical chunk (l % (kBK/16)) ^ swz_key(row).  Rows past M (or
  // N) re-read the last row: they only feed outputs that are never stored.
  constexpr int kRowsPerDma = 64 * 16 / kBK;     // 16 or 8
  constexpr int kChunks = kBK / 16;
  const int lrow = lane / kChunks;
  const int pchunk = lane % kChunks;
  uint32_t aoff[TL::ALOADS], boff[TL::BLOADS];
#pragma unroll
  for (int j = 0; j < TL::ALOADS; ++j) {
    const int r = (j * (kThreads / 64) + wave) * kRowsPerDma + lrow;   // LDS row in the stage
    int gm = m0 + r;
    gm = gm < M ? gm : M - 1;
    aoff[j] = (uint32_t)(gm * K + (pchunk ^ swz_key<kBK>(r)) * 16);
  }
#pragma unroll
  for (int j = 0; j < TL::BLOADS; ++j) {
    const int r = (j * (kThreads / 64) + wave) * kRowsPerDma + lrow;
    int gn = n0 + r;
    gn = gn < N ? gn : N - 1;
    boff[j] = (uint32_t)(gn * K + (pchunk ^ swz_key<kBK>(r)) * 16);
  }
  const int swave = __builtin_amdgcn_readfirstlane(wave);
  auto dma = [&](uint8_t* sa, uint8_t* sb, int k0) {
    const uint8_t* abase = g.a + k0;
    const uint8_t* bbase = g.b + k0;
#pragma unroll
    for (int j = 0; j < TL::ALOADS; ++j)
      dma16(abase, aoff[j], sa + (j * (kThreads / 64) + swave) * kRowsPerDma * kBK);
#pragma unroll
    for (int j = 0; j < TL::BLOADS; ++j)
      dma16(bbase, boff[j], sb + (j * (kThreads / 64) + swave) * kRowsPerDma * kBK);
  };
  // DMA instruction k (0 .. LOADS-1) of a stage: A rows first, then B rows
  auto dma_one = [&](int k, uint8_t* sa, uint8_t* sb, int k0) {
    if (k < TL::ALOADS)
      dma16(g.a + k0, aoff[k], sa + (k * (kThreads / 64) + swave) * kRowsPerDma * kBK);
    else
      dma16(g.b + k0, boff[k - TL::ALOADS], sb + ((k - TL::ALOADS) * (kThreads / 64) + swave) * kRowsPerDma * kBK);
  };
  // Register loader for a last stage that K does not fill: chunks past K are
  // zero so they add nothing to the dot products.
  auto tail = [&](uint8_t* sa, uint8_t* sb, int k0) {
#pragma unroll
    for (int j = 0; j < TL::ALOADS; ++j) {
      const int i = tid + j * kThreads, row = i / kChunks, c = i % kChunks;
      const int gm = (m0 + row) < M ? (m0 + row) : M - 1;
      const int gk = k0 + c * 16;
      *(v4i*)(sa + swz<kBK>(row, c)) = gk < K ? *(const v4i*)(g.a + gm * K + gk) : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < TL::BLOADS; ++j) {
      const int i = tid + j * kThreads, row = i / kChunks, c = i % kChunks;
      const int gn = (n0 + row) < N ? (n0 + row) : N - 1;
      const int gk = k0 + c * 16;
      *(v4i*)(sb + swz<kBK>(row, c)) = gk < K ? *(const v4i*)(g.b + gn * K + gk) : v4i{0, 0, 0, 0};
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
  const int loff = MM::template lane_off<kBK>(lane);
  // Fragments live in two register sets: while the MFMAs of one k-step run,
  // the LDS reads of the next k-step (or, across a stage boundary, of the
  // next stage's first k-step) go to the other set.
  typename MM::Op fa[2][TL::FM], fb[2][TL::FN];
  auto load_frag = [&](auto SET, int f, const uint8_t* As, const uint8_t* Bs, int ks) {
    constexpr int st = decltype(SET)::value;
    if (f < TL::FM) fa[st][f] = MM::load(As + arow + f * 32 * kBK, loff, ks);
    else fb[st][f - TL::FM] = MM::load(Bs + brow + (f - TL::FM) * 32 * kBK, loff, ks);
  };
  auto load_frags = [&](auto SET, const uint8_t* As, const uint8_t* Bs, int ks) {
#pragma unroll
    for (int f = 0; f < TL::FM + TL::FN; ++f) load_frag(SET, f, As, Bs, ks);
  };
  auto mfmas = [&](auto SET) {
    constexpr int st = decltype(SET)::value;
#pragma unroll
    for (int i = 0; i < TL::FM; ++i)
#pragma unroll
      for (int j = 0; j < TL::FN; ++j) acc[i][j] = MM::mma(fb[st][j], fa[st][i], acc[i][j]);
  };
  // One k-step's MFMAs on register set CUR with other work spread between
  // them, in this order (sched_barrier pins it): after MFMA t come the LDS
  // reads of fragments [t*F/NM, (t+1)*F/NM) into set NXT (if pf) and DMA
  // instructions [t*L/NM, (t+1)*L/NM) of a later stage (if dm).  Issued in a
  // burst, the DMA instructions stall the wave on the vector-memory queue
  // while the MFMA pipe runs dry; spread out, each waits behind an MFMA.
  // pf and dm are compile-time constants in the steady-state loop; in the
  // last stages only these slots, never the MFMAs, are conditional.
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using T = std::true_type;
  using F = std::false_type;
  auto step = [&](auto CUR, auto NXT, bool pf, bool dm, const uint8_t* xa, const uint8_t* xb, int xks,
                  uint8_t* da, uint8_t* db, int dk0) {
    constexpr int cs = decltype(CUR)::value;
    constexpr int NM = TL::FM * TL::FN, NF = TL::FM + TL::FN, NL = TL::LOADS;
#pragma unroll
    for (int t = 0; t < NM; ++t) {
      const int i = t / TL::FN, j = t % TL::FN;
      acc[i][j] = MM::mma(fb[cs][j], fa[cs][i], acc[i][j]);
      if (pf) {
#pragma unroll
        for (int f = (t * NF + NM - 1) / NM; f < ((t + 1) * NF + NM - 1) / NM; ++f) load_frag(NXT, f, xa, xb, xks);
      }
      if (dm) {
#pragma unroll
        for (int k = (t * NL + NM - 1) / NM; k < ((t + 1) * NL + NM - 1) / NM; ++k) dma_one(k, da, db, dk0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // ---- main loop.  Stage s lives in buffer s % 4; its DMA is issued during
  // stage s-4's last k-step.  Before stage s+1's fragments are read, each wave
  // waits until at most the DMA of stages s+2, s+3 is outstanding (its own
  // loads retire in order) and has finished its own LDS reads of stage s;
  // the barrier then makes every wave's copy of stage s+1 visible and proves
  // that buffer s % 4 is free for the DMA of stage s+4.
  auto wait_stage = [&](int s, bool steady) {
    const int later = steady || (nfull - 1 - s) >= 2 ? 2 : nfull - 1 - s;   // stages issued after s
    if (later >= 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * TL::LOADS) : "memory");
    else if (later == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(TL::LOADS) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // A bare s_barrier: __syncthreads() adds a workgroup release fence, which
    // waits for every LDS write in flight, the DMA of later stages included.
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // One stage whose first k-step's fragments are in register set P.  STEADY:
  // the next stage exists and so does stage s+4 (no run-time tests).
  auto stage = [&](auto PC, auto STEADY, int s, uint8_t* ca, uint8_t* cb, const uint8_t* xa,
                   const uint8_t* xb) {
    constexpr int P = decltype(PC)::value;
#pragma unroll
    for (int ks = 0; ks + 1 < KS; ++ks) {
      if ((P + ks) & 1) step(S1{}, S0{}, true, false, ca, cb, ks + 1, ca, cb, 0);
      else step(S0{}, S1{}, true, false, ca, cb, ks + 1, ca, cb, 0);
    }
    constexpr int last = (P + KS - 1) & 1;
    using CUR = std::integral_constant<int, last>;
    using NXT = std::integral_constant<int, last ^ 1>;
    // This wave's LDS reads of stage s are complete (issued a k-step ago).
    // As an s_waitcnt the compiler sees, it also tells the compiler's own
    // wait insertion that nothing is pending past this point.
    __builtin_amdgcn_s_waitcnt(kLgkmcnt0);
    const bool nxt = decltype(STEADY)::value || s + 1 < nfull;
    const bool ahead = decltype(STEADY)::value || s + 4 < nfull;
    if (nxt) wait_stage(s + 1, decltype(STEADY)::value);
    step(CUR{}, NXT{}, nxt, ahead, xa, xb, 0, ca, cb, (s + 4) * kBK);
  };
  constexpr int P1 = KS & 1, P2 = (2 * KS) & 1, P3 = (3 * KS) & 1;
  using C1 = std::integral_constant<int, P1>;
  using C2 = std::integral_constant<int, P2>;
  using C3 = std::integral_constant<int, P3>;
  if (nfull > 0) dma(sa0, sb0, 0);
  if (nfull > 1) dma(sa1, sb1, kBK);
  if (nfull > 2) dma(sa2, sb2, 2 * kBK);
  if (nfull > 0) {
    wait_stage(0, false);
    if (nfull > 3) dma(sa3, sb3, 3 * kBK);
    load_frags(S0{}, sa0, sb0, 0);
  }
  int kt = 0;
  // steady state: stages kt .. kt+3 all have a stage four ahead
  for (; kt + 8 <= nfull; kt += 4) {          // single exit: the accumulators stay in place
    stage(S0{}, T{}, kt, sa0, sb0, sa1, sb1);
    stage(C1{}, T{}, kt + 1, sa1, sb1, sa2, sb2);
    stage(C2{}, T{}, kt + 2, sa2, sb2, sa3, sb3);
    stage(C3{}, T{}, kt + 3, sa3, sb3, sa0, sb0);
  }
  // the last (up to 7) stages
  if (kt + 4 <= nfull) {
    stage(S0{}, F{}, kt, sa0, sb0, sa1, sb1);
    stage(C1{}, F{}, kt + 1, sa1, sb1, sa2, sb2);
    stage(C2{}, F{}, kt + 2, sa2, sb2, sa3, sb3);
    stage(C3{}, F{}, kt + 3, sa3, sb3, sa0, sb0);
    kt += 4;
  }
  if (kt < nfull) stage(S0{}, F{}, kt, sa0, sb0, sa1, sb1);
  if (kt + 1 < nfull) stage(C1{}, F{}, kt + 1, sa1, sb1, sa2, sb2);
  if (kt + 2 < nfull) stage(C2{}, F{}, kt + 2, sa2, sb2, sa3, sb3);
  // ---- the partial last stage, through registers, in buffer nfull % 4 (last
  // read by stage nfull - 4, long finished)
  if (ragged) {
    const int b = nfull & 3;
    uint8_t* ta = b == 0 ? sa0 : b == 1 ? sa1 : b == 2 ? sa2 : sa3;
    uint8_t* tb = b == 0 ? sb0 : b == 1 ? sb1 : b == 2 ? sb2 : sb3;
    __syncthreads();
    tail(ta, tb, nfull * kBK);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      load_frags(S0{}, ta, tb, ks);
      mfmas(S0{});
    }
  }

  // ---- epilogue.  The weight fragment is the MFMA's first operand, so
  // fragment (i, j) holds D[n][m]: register r of lane l is output
  // m = mw + i*32 + l%32, n = nw + j*32 + out_row(r, l); registers 4q..4q+3
  // are four consecutive n of one m.  Each wave moves one 32-row slab at a
  // time through a padded LDS staging tile as raw accumulators (16-byte
  // writes, no arithmetic), reads it back row-contiguous -- lane l then
  // always holds the same 8 columns, 8*(l % (TN/8)) .. +7, whose factors it
  // keeps in registers -- applies the dequantization there, and stores 16
  // bytes per lane (two rows of 256 bytes per instruction at TN = 128).
  const int mw = wm * TL::TM, nw = wn * TL::TN;
  const int lm = lane & 31, lh = lane >> 5;
  constexpr int kFacBytes = ((2 * BM + 3 * BN) * 4 + 15) / 16 * 16;
  float* const f_sx = (float*)smem;                     // [BM]
  int* const f_rs = (int*)(f_sx + BM);                  // [BM]
  float* const f_sb = (float*)(f_rs + BM);              // [BN]
  int* const f_zi = (int*)(f_sb + BN);                  // [BN] zero points (exact integers)
  float* const f_bb = (float*)(f_zi + BN);              // [BN]
  __syncthreads();                                      // the main loop's LDS reads are done
  if (tid < BM) { f_sx[tid] = pf_sx; f_rs[tid] = pf_rs; }
  if (tid < BN) { f_sb[tid] = pf_sb; f_zi[tid] = pf_zi; f_bb[tid] = pf_bb; }
  __syncthreads();

  if constexpr (KIND == GEMM_INT8_DECOMP) {
    // LLM.int8: dequantize the int8 part in place (the fp32 value replaces
    // the int32 in the same registers), then add the outlier flow with
    // v_mfma_f32_32x32x16_f16 (same 32 x 32 output layout, weights first)
    // whose accumulator input is that value.
#pragma unroll
    for (int i = 0; i < TL::FM; ++i) {
      const int ml = mw + i * 32 + lm, m = m0 + ml;
      const float sx = f_sx[ml];
      const int rs = f_rs[ml];
#pragma unroll
      for (int j = 0; j < TL::FN; ++j)
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const int nl = nw + j * 32 + out_row(r, lane), n = n0 + nl;
          const int a = acc[i][j][r];
          if (g.acc_out && m < M && n < N) g.acc_out[m * N + n] = a;
          acc[i][j][r] = __float_as_int((sx * f_sb[nl]) * (float)(a - f_zi[nl] * rs));
        }
    }
    // the prefetched count and panels are first used here (the empty asm
    // keeps their uses from being hoisted next to their loads)
    asm volatile("" : "+v"(pf_cnt));
    const int cnt = pf_cnt;
    static_assert(kPanelCols == 16, "one v_mfma_f32_32x32x16_f16 step per panel");
    const int kg = lane >> 5;                          // 8-column group of the 16-column step
    auto outlier_mfmas = [&](const v8h* xo, const v8h* wo) {
#pragma unroll
      for (int i = 0; i < TL::FM; ++i)
#pragma unroll
        for (int j = 0; j < TL::FN; ++j) {
          v16f c = __builtin_bit_cast(v16f, acc[i][j]);
          c = __builtin_amdgcn_mfma_f32_32x32x16_f16(wo[j], xo[i], c, 0, 0, 0);
          acc[i][j] = __builtin_bit_cast(v16i, c);
        }
    };
    if (cnt > 0) {
      // the first kPanelCols outlier columns, from the quantizer's panels
      // (zeros past the count)
      v8h xo[TL::FM], wo[TL::FN];
#pragma unroll
      for (int i = 0; i < TL::FM; ++i) {
        asm volatile("" : "+v"(pf_xo[i]));
        xo[i] = __builtin_bit_cast(v8h, pf_xo[i]);
      }
#pragma unroll
      for (int j = 0; j < TL::FN; ++j) {
        asm volatile("" : "+v"(pf_wo[j]));
        wo[j] = __builtin_bit_cast(v8h, pf_wo[j]);
      }
      outlier_mfmas(xo, wo);
    }
    for (int kc = kPanelCols; kc < cnt; kc += 16) {
      int col[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int jj = kc + kg * 8 + e;
        col[e] = jj < cnt ? g.out_idx[jj] : -1;
      }
      // Every load is issued unconditionally, at a clamped address, and all
      // of them before any is used; each value is zeroed afterwards where its
      // column or row does not exist.  (Written as `cond ? load : 0`, the
      // compiler moved each load under a branch and waited for it before
      // issuing the next: 8 + 8 round trips in a row.)  The empty asm
      // statements take every loaded value after the last load is issued.
      uint32_t xr[TL::FM][8], wr[TL::FN][8];
#pragma unroll
      for (int i = 0; i < TL::FM; ++i) {
        const int m = m0 + mw + i * 32 + lm;
        const int mc = m < M ? m : M - 1;
#pragma unroll
        for (int e = 0; e < 8; ++e) xr[i][e] = g.x_f16[mc * K + (col[e] >= 0 ? col[e] : 0)];
      }
#pragma unroll
      for (int j = 0; j < TL::FN; ++j) {
        const int n = n0 + nw + j * 32 + lm;
        const int ncl = n < N ? n : N - 1;
#pragma unroll
        for (int e = 0; e < 8; ++e) wr[j][e] = (uint32_t)(uint8_t)g.b[ncl * K + (col[e] >= 0 ? col[e] : 0)];
      }
#pragma unroll
      for (int i = 0; i < TL::FM; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) asm volatile("" : "+v"(xr[i][e]));
#pragma unroll
      for (int j = 0; j < TL::FN; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) asm volatile("" : "+v"(wr[j][e]));
      v8h xo[TL::FM], wo[TL::FN];
#pragma unroll
      for (int i = 0; i < TL::FM; ++i) {
        const int m = m0 + mw + i * 32 + lm;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          xo[i][e] = (col[e] >= 0 && m < M) ? __builtin_bit_cast(_Float16, (uint16_t)xr[i][e]) : (_Float16)0.0f;
      }
#pragma unroll
      for (int j = 0; j < TL::FN; ++j) {
        const int nl = nw + j * 32 + lm, n = n0 + nl;
        const bool nok = n < N;
        const float sb = f_sb[nl], zb = (float)f_zi[nl];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const _Float16 w = outlier_weight_f16(sb, (int8_t)(uint8_t)wr[j][e], zb);
          wo[j][e] = (col[e] >= 0 && nok) ? w : (_Float16)0.0f;
        }
      }
      outlier_mfmas(xo, wo);
    }
  }

  // staging: per wave 32 rows of TN raw 32-bit values, pitch TN*4 + 16 bytes
  // (16-byte aligned; the 16 rows of one 16-byte write fall in 16 different
  // bank quarters)
  constexpr int kPitch = TL::TN * 4 + 16;
  constexpr int LPR = TL::TN / 8;                       // readback lanes per row
  constexpr int RPI = 64 / LPR;                         // rows per readback instruction
  static_assert(kFacBytes + NW * 32 * kPitch <= kStages * kStageBytes, "epilogue staging does not fit");
  uint8_t* const stg = smem + kFacBytes + wave * 32 * kPitch;
  const int rc = lane % LPR, rr = lane / LPR;
  const int ncl = nw + 8 * rc;                          // first of the lane's 8 columns in the tile
  const int n = n0 + ncl;
  // the lane's column factors
  const v4f csb0 = *(const v4f*)(f_sb + ncl), csb1 = *(const v4f*)(f_sb + ncl + 4);
  const v4f cbb0 = *(const v4f*)(f_bb + ncl), cbb1 = *(const v4f*)(f_bb + ncl + 4);
  const v4i czi0 = *(const v4i*)(f_zi + ncl), czi1 = *(const v4i*)(f_zi + ncl + 4);
  const float csb[8] = {csb0[0], csb0[1], csb0[2], csb0[3], csb1[0], csb1[1], csb1[2], csb1[3]};
  const float cbb[8] = {cbb0[0], cbb0[1], cbb0[2], cbb0[3], cbb1[0], cbb1[1], cbb1[2], cbb1[3]};
  const int czi[8] = {czi0[0], czi0[1], czi0[2], czi0[3], czi1[0], czi1[1], czi1[2], czi1[3]};
  // acc - Z rowsum as one full-rate 24-bit multiply-add: |Z| <= 128 and
  // |rowsum| <= 127 K < 2^23 (K <= 65536), and the product fits 32 bits
  // (a full 32-bit multiply issues at a quarter of the rate)
  auto zcorr = [](int acc, int z, int rs) { return acc + __mul24(-z, rs); };
  constexpr int ES = YDT == DT_F32 ? 4 : 2;
  const bool vec = (N & 7) == 0;                        // 8-column groups start 16-byte aligned
  const bool full = vec && m0 + BM <= M && n0 + BN <= N; // an interior tile: no row or column past Y
#pragma unroll
  for (int i = 0; i < TL::FM; ++i) {
#pragma unroll
    for (int j = 0; j < TL::FN; ++j)
#pragma unroll
      for (int q = 0; q < NR / 4; ++q) {
        const int cl = j * 32 + 8 * q + 4 * lh;
        *(v4i*)(stg + lm * kPitch + cl * 4) = v4i{raw32(acc[i][j][4 * q]), raw32(acc[i][j][4 * q + 1]),
                                                  raw32(acc[i][j][4 * q + 2]), raw32(acc[i][j][4 * q + 3])};
      }
    // the wave's own staging writes precede these reads (LDS is in order).
    // All of the slab's readback reads and row factors are issued before any
    // is used, so their LDS latency overlaps.
    constexpr int TI = 32 / RPI;                        // readback instructions per slab
    v4i ra[TI], rb[TI];
    float rsx[TI];
    int rrs[TI];
#pragma unroll
    for (int t = 0; t < TI; ++t) {
      const int row = t * RPI + rr;
      ra[t] = *(const v4i*)(stg + row * kPitch + rc * 32);
      rb[t] = *(const v4i*)(stg + row * kPitch + rc * 32 + 16);
      rsx[t] = f_sx[mw + i * 32 + row];
      rrs[t] = KIND == GEMM_INT8 ? f_rs[mw + i * 32 + row] : 0;
    }
    // one output row of the slab.  CHK: bounds and 16-byte alignment are
    // checked per row (a tile at the edge of Y); ACC: the INT32 accumulator
    // may be stored too.  An interior tile without the accumulator output
    // runs without per-row tests.
    auto row = [&](int t, auto CHK, auto ACC) __attribute__((always_inline)) {
      constexpr bool chk = decltype(CHK)::value;
      const int m = m0 + mw + i * 32 + t * RPI + rr;
      const bool ok = !chk || (m < M && n < N);
      const int a[8] = {ra[t][0], ra[t][1], ra[t][2], ra[t][3], rb[t][0], rb[t][1], rb[t][2], rb[t][3]};
      const size_t o = (size_t)(uint32_t)(m * N + n);
      if constexpr (KIND == GEMM_INT8 && decltype(ACC)::value) {
        if (g.acc_out && ok) {
          if (!chk || vec) {
            *(v4i*)(g.acc_out + o) = ra[t];
            *(v4i*)(g.acc_out + o + 4) = rb[t];
          } else {
            for (int e = 0; e < 8 && n + e < N; ++e) g.acc_out[o + e] = a[e];
          }
        }
      }
      const float sx = rsx[t];
      if constexpr (YDT == DT_I8) {
        // requantized INT8 output (int8 GEMM only): the codes are decided in
        // float64 exactly as the definition states
        if (!ok) return;
        int qv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[e] = requant_i8(sx, csb[e], zcorr(a[e], czi[e], rrs[t]), cbb[e], g.y_inv);
        int8_t* yq = (int8_t*)g.y + o;
        if (!chk || vec) {
          *(v2i*)yq = v2i{(int)pack_lo_bytes(qv[0], qv[1], qv[2], qv[3]), (int)pack_lo_bytes(qv[4], qv[5], qv[6], qv[7])};
        } else {
          for (int e = 0; e < 8 && n + e < N; ++e) yq[e] = (int8_t)qv[e];
        }
      } else {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if constexpr (KIND == GEMM_INT8) {
            v[e] = (sx * csb[e]) * (float)zcorr(a[e], czi[e], rrs[t]) + cbb[e];
          } else if constexpr (KIND == GEMM_FP8) {
            v[e] = __int_as_float(a[e]) * (sx * csb[e]) + cbb[e];
          } else {
            v[e] = __int_as_float(a[e]) + cbb[e];
          }
        }
        if (!ok) return;
        if (!chk || vec) {
          // the output is written once and not read back here: non-temporal stores
          if constexpr (YDT == DT_F32) {
            v4i* yp = (v4i*)((float*)g.y + o);
            __builtin_nontemporal_store(v4i{__float_as_int(v[0]), __float_as_int(v[1]), __float_as_int(v[2]),
                                            __float_as_int(v[3])}, yp);
            __builtin_nontemporal_store(v4i{__float_as_int(v[4]), __float_as_int(v[5]), __float_as_int(v[6]),
                                            __float_as_int(v[7])}, yp + 1);
          } else {
            v4i pk;
#pragma unroll
            for (int e = 0; e < 4; ++e) pk[e] = (int)pack2_out<YDT>(v[2 * e], v[2 * e + 1]);
            __builtin_nontemporal_store(pk, (v4i*)((uint16_t*)g.y + o));
          }
        } else {
          for (int e = 0; e < 8 && n + e < N; ++e) store_out<YDT>(g.y, o + e, v[e]);
        }
      }
    };
    using Tt = std::true_type;
    using Ft = std::false_type;
    if (full && !g.acc_out) {
#pragma unroll
      for (int t = 0; t < TI; ++t) row(t, Ft{}, Ft{});
    } else {
#pragma unroll
      for (int t = 0; t < TI; ++t) row(t, Tt{}, Tt{});
    }
  }
  (void)ES;
}

// Output types: int8 GEMM f32 / f16 / bf16; the outlier flow f16 (the
// decomposition's output is fp16); fp8 bf16.
template <int BM, int BN, int KIND>
hipError_t launch_tiles(const GemmArgs& g, int ydt, hipStream_t st) {
  // The int8 tiles of 256 x 256, 128 x 128 and 64 x 128 run 8 waves (two per
  // SIMD: 128 x 64, 64 x 32 and 32 x 32 each), so one wave's stalls on the DMA
  // issue and its fragment reads are covered by the other's MFMAs; the fp8
  // operands are twice as wide and spill at that register budget on 256 x 256
  // (on 128 x 128 eight fp8 waves measured no faster)
  constexpr int NW = KIND != GEMM_FP8 && ((BM == 256 && BN == 256) || (BM == 64 && BN == 128) || (BM == 128 && BN == 128))
                         ? 8 : 4;
  const int64_t ntm = (g.M + BM - 1) / BM, ntn = (g.N + BN - 1) / BN;
  dim3 grid((unsigned)(ntm * ntn)), block(64 * NW);
  if constexpr (KIND == GEMM_INT8) {
    switch (ydt) {
      case DT_I8: k_gemm<BM, BN, KIND, DT_I8, NW><<<grid, block, 0, st>>>(g); break;
      case DT_F32: k_gemm<BM, BN, KIND, DT_F32, NW><<<grid, block, 0, st>>>(g); break;
      case DT_F16: k_gemm<BM, BN, KIND, DT_F16, NW><<<grid, block, 0, st>>>(g); break;
      default: k_gemm<BM, BN, KIND, DT_BF16, NW><<<grid, block, 0, st>>>(g); break;
    }
  } else if constexpr (KIND == GEMM_INT8_DECOMP) {
    if (ydt != DT_F16) return hipErrorInvalidValue;
    k_gemm<BM, BN, KIND, DT_F16, NW><<<grid, block, 0, st>>>(g);
  } else {
    if (ydt != DT_BF16) return hipErrorInvalidValue;
    k_gemm<BM, BN, KIND, DT_BF16, NW><<<grid, block, 0, st>>>(g);
  }
  return hipGetLastError();
}

template <int KIND>
hipError_t launch_kind(const GemmArgs& g, int ydt, hipStream_t st) {
  int bm = 0, bn = 0;
  gemm_tile((GemmKind)KIND, g.M, g.N, &bm, &bn);
  if constexpr (KIND != GEMM_INT8_DECOMP) {
    if (bm == 256) return launch_tiles<256, 256, KIND>(g, ydt, st);
  }
  if (bm == 128) return launch_tiles<128, 128, KIND>(g, ydt, st);
  if (bn == 128) return launch_tiles<64, 128, KIND>(g, ydt, st);
  return launch_tiles<64, 64, KIND>(g, ydt, st);
}

}  // namespace

// Pick the largest tile that still gives most of the 256 CUs a workgroup.
void gemm_tile(GemmKind kind, int64_t M, int64_t N, int* bm, int* bn) {
  auto tiles = [&](int64_t tm, int64_t tn) { return ((M + tm - 1) / tm) * ((N + tn - 1) / tn); };
  // the outlier flow needs the accumulators in VGPRs: no 256 x 256 tile there
  if (kind != GEMM_INT8_DECOMP && tiles(256, 256) >= 192) { *bm = 256; *bn = 256; return; }
  if (tiles(128, 128) >= 192) { *bm = 128; *bn = 128; return; }
  // e.g. the LLM.int8 shape 512 x 4096: one round of 256 tiles, two
  // independent accumulators per wave
  if (tiles(64, 128) >= 192) { *bm = 64; *bn = 128; return; }
  *bm = 64; *bn = 64;
}

hipError_t launch_gemm_fp8_grouped(const GemmArgs& g, hipStream_t st) {
  // tile size from the mean rows per group; the grid bounds the tile count:
  // sum_e ceil(M_e / BM) <= M / BM + groups.  Each group ends in a partial
  // tile, and with 256 x 256 tiles a mean of 512 rows leaves about 1.25
  // rounds of tiles on 256 CUs: there 128 x 128 is faster (98 against 104 us
  // for 8 experts of 4096 x 4096, K = 4096); from a mean of 768 rows on the
  // larger tile wins (113 against 133 us, and 296 against 358 at 2048)
  const int64_t mean = g.M / (g.groups > 0 ? g.groups : 1);
  auto grid_for = [&](int bm, int bn) {
    return dim3((unsigned)(((g.M + bm - 1) / bm + g.groups) * ((g.N + bn - 1) / bn)));
  };
  if (mean >= 768)
    k_gemm<256, 256, GEMM_FP8, DT_BF16, 4, true><<<grid_for(256, 256), 256, 0, st>>>(g);
  else if (mean >= 128)
    k_gemm<128, 128, GEMM_FP8, DT_BF16, 4, true><<<grid_for(128, 128), 256, 0, st>>>(g);
  else
    k_gemm<64, 128, GEMM_FP8, DT_BF16, 4, true><<<grid_for(64, 128), 256, 0, st>>>(g);
  return hipGetLastError();
}

hipError_t launch_gemm(GemmKind kind, const GemmArgs& g, int ydt, hipStream_t st) {
  switch (kind) {
    case GEMM_INT8: return launch_kind<GEMM_INT8>(g, ydt, st);
    case GEMM_INT8_DECOMP: return launch_kind<GEMM_INT8_DECOMP>(g, ydt, st);
    default: return launch_kind<GEMM_FP8>(g, ydt, st);
  }
}

}  // namespace q8
