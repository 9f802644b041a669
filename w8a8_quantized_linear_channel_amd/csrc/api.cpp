// C ABI of libq8: argument validation, workspace carving and kernel dispatch.
// Every check that needs no device runs first, so argument errors are
// reported before any HIP call (and can be exercised on a machine without a
// GPU); then the device of the stream is checked once per device and cached.
#include "q8.h"
#include "q8_bench.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>

#include "q8_bench_kernels.hpp"
#include "q8_group.hpp"
#include "q8_kernels.hpp"
#include "q8_linear_impl.hpp"

namespace {

constexpr int64_t kMaxK = 65536;          // keeps acc - Z*rowsum inside int32 (|.| <= 32512 K)
constexpr int64_t kMaxRows = (1LL << 31) - 1;
constexpr size_t kAlign = 256;
constexpr int64_t kMaxGroups = 1024;            // experts of one grouped call (the kernels' bound)

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3) == 0; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool valid_dtype(int d) { return d == Q8_F32 || d == Q8_F16 || d == Q8_BF16; }

// M rows of K; min_m = 0 admits an empty batch of activations
q8_status check_mk(int64_t M, int64_t K, int64_t min_m = 1) {
  if (M < min_m || K < 1 || M > kMaxRows) return Q8_ERR_BAD_SHAPE;
  if (K % 16 != 0 || K > kMaxK) return Q8_ERR_BAD_SHAPE;
  return Q8_OK;
}

// M activation rows (0: an empty batch), N weight rows, K features
q8_status check_mnk(int64_t M, int64_t N, int64_t K) {
  q8_status s = check_mk(M, K, 0);
  if (s != Q8_OK) return s;
  if (N < 1 || N > kMaxRows) return Q8_ERR_BAD_SHAPE;
  // the GEMM indexes its operands and output with 32-bit offsets
  if (M * K > kMaxRows || N * K > kMaxRows || M * N > kMaxRows) return Q8_ERR_BAD_SHAPE;
  return Q8_OK;
}

// Bump allocator over the caller's workspace; every piece 256-byte aligned.
struct Carve {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off = (off + bytes + kAlign - 1) / kAlign * kAlign;
    return o;
  }
};

// The int8 product and epilogue on quantized activations: the streaming GEMV
// for decode-sized M, the MFMA GEMM tiles above.
hipError_t int8_on_codes(const int8_t* xq, const float* xs, const int32_t* rs, int64_t M, int64_t K,
                         const int8_t* wq, const float* w_scale, const float* w_zp, int64_t N, const float* bias,
                         void* y, int y_dtype, int32_t* acc_out, hipStream_t st, double y_inv = 0.0) {
  if (M <= q8::kGemvMaxM)
    return q8::launch_gemv_q8(xq, xs, rs, M, K, wq, w_scale, w_zp, N, bias, y, y_dtype, acc_out, st, y_inv);
  q8::GemmArgs g{};
  g.a = reinterpret_cast<const uint8_t*>(xq);
  g.b = reinterpret_cast<const uint8_t*>(wq);
  g.a_scale = xs;
  g.a_rowsum = rs;
  g.b_scale = w_scale;
  g.b_zp = w_zp;
  g.bias = bias;
  g.y = y;
  g.acc_out = acc_out;
  g.M = M;
  g.N = N;
  g.K = K;
  g.y_inv = y_inv;
  return q8::launch_gemm(q8::GEMM_INT8, g, y_dtype, st);
}

struct LinearWs { size_t xq, xs, rs, total; };

// Static path: the codes, the per-row copy of the static scale and the code
// sums always pass through the workspace.
LinearWs static_ws(int64_t M, int64_t K) {
  Carve c;
  LinearWs w;
  w.xq = c.take((size_t)M * K);
  w.xs = c.take((size_t)M * 4);
  w.rs = c.take((size_t)M * 4);
  w.total = c.off;
  return w;
}
LinearWs linear_ws(int64_t M, int64_t K) {
  LinearWs w{0, 0, 0, 0};
  if (M <= q8::kGemvFusedMaxM) return w;   // fused decode path: the codes stay in LDS, no scratch
  Carve c;
  w.xq = c.take((size_t)M * K);
  w.xs = c.take((size_t)M * 4);
  w.rs = c.take((size_t)M * 4);
  w.total = c.off;
  return w;
}

// Per-group path: codes, scales and the group code sums [K / group, M], sized
// for the smallest group (64); none for the fused decode path.
struct GroupedWs { size_t xq, xs, gs, total; };
GroupedWs grouped_ws(int64_t M, int64_t K) {
  GroupedWs w{0, 0, 0, 0};
  if (M <= q8::kGemvFusedMaxM) return w;
  Carve c;
  w.xq = c.take((size_t)M * K);
  w.xs = c.take((size_t)M * 4);
  w.gs = c.take((size_t)M * (K / 64) * 4);
  w.total = c.off;
  return w;
}
bool valid_group(int64_t group, int64_t K) { return (group == 64 || group == 128) && K % group == 0; }

// LLM.int8: codes, scales, row sums, column flags, outlier list and count,
// and the fp16 panels of the first kPanelCols outlier columns of X and W.
struct DecompWs { size_t xq, xs, rs, flags, idx, cnt, xp, wp, total; };
DecompWs decomp_ws(int64_t M, int64_t N, int64_t K) {
  if (M == 0) return DecompWs{};   // an empty batch needs no scratch
  Carve c;
  DecompWs w;
  w.xq = c.take((size_t)M * K);
  w.xs = c.take((size_t)M * 4);
  w.rs = c.take((size_t)M * 4);
  w.flags = c.take((size_t)K);
  w.idx = c.take((size_t)K * 4);
  w.cnt = c.take(4);
  w.xp = c.take((size_t)M * q8::kPanelCols * 2);
  w.wp = c.take((size_t)N * q8::kPanelCols * 2);
  w.total = c.off;
  return w;
}

struct Fp8Ws { size_t xq, xs, total; };
Fp8Ws fp8_ws(int64_t M, int64_t K) {
  Carve c;
  Fp8Ws w;
  w.xq = c.take((size_t)M * K);
  w.xs = c.take((size_t)M * 4);
  w.total = c.off;
  return w;
}

// ---- device check: gfx950 only, cached per device
constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];   // 0 unknown, 1 gfx950, 2 other

q8_status device_of(hipStream_t st, int* dev) {
  if (st != nullptr) {
    if (hipStreamGetDevice(st, dev) != hipSuccess) return Q8_ERR_DEVICE;
  } else if (hipGetDevice(dev) != hipSuccess) {
    return Q8_ERR_DEVICE;
  }
  return (*dev >= 0 && *dev < kMaxDevices) ? Q8_OK : Q8_ERR_DEVICE;
}

q8_status check_device(hipStream_t st) {
  int dev = -1;
  q8_status s = device_of(st, &dev);
  if (s != Q8_OK) {
    (void)hipGetLastError();   // do not leave a sticky error for the caller
    return s;
  }
  int state = g_dev_state[dev].load(std::memory_order_relaxed);
  if (state == 0) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) {
      (void)hipGetLastError();
      return Q8_ERR_DEVICE;
    }
    state = (std::strncmp(p.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_dev_state[dev].store(state, std::memory_order_relaxed);
  }
  return state == 1 ? Q8_OK : Q8_ERR_DEVICE;
}

// Optional (Q8_DEBUG_VALIDATE=1): every pointer must be device memory of the
// stream's device.
bool debug_validate() {
  static const bool on = [] {
    const char* e = std::getenv("Q8_DEBUG_VALIDATE");
    return e != nullptr && e[0] == '1';
  }();
  return on;
}

q8_status check_ptrs(hipStream_t st, std::initializer_list<const void*> ptrs) {
  if (!debug_validate()) return Q8_OK;
  int dev = -1;
  if (device_of(st, &dev) != Q8_OK) return Q8_ERR_DEVICE;
  for (const void* p : ptrs) {
    if (p == nullptr) continue;
    hipPointerAttribute_t a;
    if (hipPointerGetAttributes(&a, p) != hipSuccess) {
      (void)hipGetLastError();
      return Q8_ERR_BAD_ARG;
    }
    if (a.type != hipMemoryTypeDevice || a.device != dev) return Q8_ERR_BAD_ARG;
  }
  return Q8_OK;
}

q8_status launched(hipError_t e) { return e == hipSuccess ? Q8_OK : Q8_ERR_LAUNCH; }

#define Q8_TRY(expr)                 \
  do {                               \
    const q8_status s_ = (expr);     \
    if (s_ != Q8_OK) return s_;      \
  } while (0)

}  // namespace

namespace q8 {

q8_status linear_check_args(const void* x, q8_dtype x_dtype, int64_t M, int64_t K, const int8_t* wq,
                            const float* w_scale, const float* w_zp, int64_t N, const float* bias, const void* y,
                            q8_dtype y_dtype, const int32_t* acc_out, size_t* workspace_needed) {
  if (!valid_dtype(x_dtype) || !valid_dtype(y_dtype)) return Q8_ERR_BAD_DTYPE;
  Q8_TRY(check_mnk(M, N, K));
  if (!wq || !w_scale || !w_zp || (M > 0 && (!x || !y))) return Q8_ERR_NULL_PTR;
  if (!aligned16(x) || !aligned16(wq) || !aligned16(w_scale) || !aligned16(w_zp) || !aligned16(y) ||
      (bias && !aligned16(bias)) || (acc_out && !aligned16(acc_out)))
    return Q8_ERR_ALIGN;
  *workspace_needed = linear_ws(M, K).total;
  return Q8_OK;
}

q8_status linear_run(const void* x, q8_dtype x_dtype, int64_t M, int64_t K, const int8_t* wq, const float* w_scale,
                     const float* w_zp, int64_t N, const float* bias, void* y, q8_dtype y_dtype, void* workspace,
                     int32_t* acc_out, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  Q8_TRY(check_device(st));
  Q8_TRY(check_ptrs(st, {x, wq, w_scale, w_zp, bias, y, workspace, acc_out}));
  if (M == 0) return Q8_OK;

  if (M <= q8::kGemvFusedMaxM)
    return launched(q8::launch_gemv_i8(x, x_dtype, M, K, wq, w_scale, w_zp, N, bias, y, y_dtype,
                                       acc_out, st));

  const LinearWs ws = linear_ws(M, K);
  char* base = static_cast<char*>(workspace);
  int8_t* xq = reinterpret_cast<int8_t*>(base + ws.xq);
  float* xs = reinterpret_cast<float*>(base + ws.xs);
  int32_t* rs = reinterpret_cast<int32_t*>(base + ws.rs);
  Q8_TRY(launched(q8::launch_quant_act_i8(x, x_dtype, M, K, xq, xs, rs, st)));
  return launched(int8_on_codes(xq, xs, rs, M, K, wq, w_scale, w_zp, N, bias, y, y_dtype, acc_out, st));
}

q8_status stream_device(void* stream, int* dev) { return device_of(static_cast<hipStream_t>(stream), dev); }

}  // namespace q8

extern "C" {

const char* q8_status_str(q8_status s) {
  switch (s) {
    case Q8_OK: return "Q8_OK";
    case Q8_ERR_NULL_PTR: return "Q8_ERR_NULL_PTR";
    case Q8_ERR_BAD_SHAPE: return "Q8_ERR_BAD_SHAPE";
    case Q8_ERR_BAD_DTYPE: return "Q8_ERR_BAD_DTYPE";
    case Q8_ERR_BAD_FORMAT: return "Q8_ERR_BAD_FORMAT";
    case Q8_ERR_BAD_ARG: return "Q8_ERR_BAD_ARG";
    case Q8_ERR_ALIGN: return "Q8_ERR_ALIGN";
    case Q8_ERR_WORKSPACE: return "Q8_ERR_WORKSPACE";
    case Q8_ERR_DEVICE: return "Q8_ERR_DEVICE";
    case Q8_ERR_LAUNCH: return "Q8_ERR_LAUNCH";
  }
  return "Q8_ERR_UNKNOWN";
}

size_t q8_workspace_bytes(q8_op op, int64_t M, int64_t N, int64_t K) {
  if (check_mnk(M, N, K) != Q8_OK) return 0;
  switch (op) {
    case Q8_OP_LINEAR: return linear_ws(M, K).total;
    case Q8_OP_DECOMP: return decomp_ws(M, N, K).total;
    case Q8_OP_FP8: return fp8_ws(M, K).total;
    case Q8_OP_STATIC: return static_ws(M, K).total;
    case Q8_OP_GROUPED: return grouped_ws(M, K).total;
  }
  return 0;
}

q8_status q8_quantize_weight(q8_format fmt, const void* w, q8_dtype w_dtype, int64_t N, int64_t K,
                             void* wq, float* w_scale, float* w_zp, void* stream) {
  if (fmt != Q8_INT8_ASYM && fmt != Q8_FP8_E4M3) return Q8_ERR_BAD_FORMAT;
  if (!valid_dtype(w_dtype)) return Q8_ERR_BAD_DTYPE;
  Q8_TRY(check_mk(N, K));
  if (!w || !wq || !w_scale) return Q8_ERR_NULL_PTR;
  if (fmt == Q8_INT8_ASYM && !w_zp) return Q8_ERR_NULL_PTR;
  if (fmt == Q8_FP8_E4M3 && w_zp) return Q8_ERR_BAD_ARG;
  if (!aligned16(w) || !aligned16(wq) || !aligned16(w_scale) || (w_zp && !aligned16(w_zp)))
    return Q8_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Q8_TRY(check_device(st));
  Q8_TRY(check_ptrs(st, {w, wq, w_scale, w_zp}));
  if (fmt == Q8_INT8_ASYM)
    return launched(q8::launch_quant_weight_i8(w, w_dtype, N, K, static_cast<int8_t*>(wq), w_scale,
                                               w_zp, st));
  return launched(q8::launch_quant_rows_fp8(w, w_dtype, N, K, INFINITY, static_cast<uint8_t*>(wq),
                                            w_scale, st));
}

q8_status q8_quantize_act(q8_format fmt, const void* x, q8_dtype x_dtype, int64_t M, int64_t K,
                          float scale_ub, void* xq, float* x_scale, int32_t* x_rowsum, void* stream) {
  if (fmt != Q8_INT8_SYM && fmt != Q8_FP8_E4M3) return Q8_ERR_BAD_FORMAT;
  if (!valid_dtype(x_dtype)) return Q8_ERR_BAD_DTYPE;
  Q8_TRY(check_mk(M, K, 0));
  if (M > 0 && (!x || !xq || !x_scale)) return Q8_ERR_NULL_PTR;
  if (fmt == Q8_FP8_E4M3) {
    if (x_rowsum) return Q8_ERR_BAD_ARG;
    if (std::isnan(scale_ub) || scale_ub <= 0.0f) return Q8_ERR_BAD_ARG;
  }
  if (!aligned16(x) || !aligned16(xq) || !aligned16(x_scale) || (x_rowsum && !aligned16(x_rowsum)))
    return Q8_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Q8_TRY(check_device(st));
  Q8_TRY(check_ptrs(st, {x, xq, x_scale, x_rowsum}));
  if (M == 0) return Q8_OK;
  if (fmt == Q8_INT8_SYM)
    return launched(q8::launch_quant_act_i8(x, x_dtype, M, K, static_cast<int8_t*>(xq),
                                            x_scale, x_rowsum, st));
  return launched(q8::launch_quant_rows_fp8(x, x_dtype, M, K, scale_ub, static_cast<uint8_t*>(xq),
                                            x_scale, st));
}

q8_status q8_linear(const void* x, q8_dtype x_dtype, int64_t M, int64_t K, const int8_t* wq,
                    const float* w_scale, const float* w_zp, int64_t N, const float* bias, void* y,
                    q8_dtype y_dtype, void* workspace, size_t workspace_bytes, int32_t* acc_out,
                    void* stream) {
  size_t need = 0;
  Q8_TRY(q8::linear_check_args(x, x_dtype, M, K, wq, w_scale, w_zp, N, bias, y, y_dtype, acc_out, &need));
  if (need > 0 && (!workspace || workspace_bytes < need)) return Q8_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return Q8_ERR_ALIGN;
  return q8::linear_run(x, x_dtype, M, K, wq, w_scale, w_zp, N, bias, y, y_dtype, workspace, acc_out, stream);
}

q8_status q8_linear_int8_decomp(const void* x, int64_t M, int64_t K, const int8_t* wq,
                                const float* w_scale, const float* w_zp, int64_t N, float threshold,
                                const float* bias, void* y, void* workspace, size_t workspace_bytes,
                                int32_t* outlier_idx, int32_t* n_outliers, int32_t* acc_out,
                                void* stream) {
  Q8_TRY(check_mnk(M, N, K));
  if (!wq || !w_scale || !w_zp || (M > 0 && (!x || !y))) return Q8_ERR_NULL_PTR;
  if (std::isnan(threshold)) return Q8_ERR_BAD_ARG;
  const DecompWs ws = decomp_ws(M, N, K);
  if (ws.total > 0 && (!workspace || workspace_bytes < ws.total)) return Q8_ERR_WORKSPACE;
  if (!aligned16(x) || !aligned16(wq) || !aligned16(w_scale) || !aligned16(w_zp) || !aligned16(y) ||
      !aligned16(workspace) || (bias && !aligned16(bias)) || (acc_out && !aligned16(acc_out)) ||
      (outlier_idx && !aligned16(outlier_idx)) || (n_outliers && !aligned16(n_outliers)))
    return Q8_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Q8_TRY(check_device(st));
  Q8_TRY(check_ptrs(st, {x, wq, w_scale, w_zp, bias, y, workspace, outlier_idx, n_outliers, acc_out}));
  if (M == 0) {
    // the outlier set of an empty batch is empty: only the count is written,
    // by the quantizer's compaction workgroup alone (no flags, no rows)
    if (n_outliers)
      return launched(q8::launch_quant_act_f16_outliers(nullptr, 0, K, nullptr, nullptr, nullptr, nullptr, nullptr,
                                                        n_outliers, nullptr, nullptr, q8::OutlierPanels{}, st));
    return Q8_OK;
  }

  char* base = static_cast<char*>(workspace);
  int8_t* xq = reinterpret_cast<int8_t*>(base + ws.xq);
  float* xs = reinterpret_cast<float*>(base + ws.xs);
  int32_t* rs = reinterpret_cast<int32_t*>(base + ws.rs);
  uint8_t* flags = reinterpret_cast<uint8_t*>(base + ws.flags);
  int32_t* idx = reinterpret_cast<int32_t*>(base + ws.idx);
  int32_t* cnt = reinterpret_cast<int32_t*>(base + ws.cnt);
  uint16_t* xp = reinterpret_cast<uint16_t*>(base + ws.xp);
  uint16_t* wp = reinterpret_cast<uint16_t*>(base + ws.wp);
  const uint16_t* xh = static_cast<const uint16_t*>(x);

  // threshold <= 0: no outlier columns (the decomposition is off)
  const bool on = threshold > 0.0f;
  if (on) Q8_TRY(launched(q8::launch_outlier_flags(xh, M, K, threshold, flags, st)));
  // the panels are needed only when there can be outlier columns
  const q8::OutlierPanels pan{wq, w_scale, w_zp, N, on ? xp : nullptr, wp};
  Q8_TRY(launched(q8::launch_quant_act_f16_outliers(xh, M, K, on ? flags : nullptr, xq, xs, rs, idx, cnt,
                                                    outlier_idx, n_outliers, pan, st)));
  q8::GemmArgs g{};
  g.a = reinterpret_cast<const uint8_t*>(xq);
  g.b = reinterpret_cast<const uint8_t*>(wq);
  g.a_scale = xs;
  g.a_rowsum = rs;
  g.b_scale = w_scale;
  g.b_zp = w_zp;
  g.bias = bias;
  g.y = y;
  g.acc_out = acc_out;
  g.M = M;
  g.N = N;
  g.K = K;
  g.x_f16 = xh;
  g.out_idx = idx;
  g.out_cnt = cnt;
  g.x_panel = xp;
  g.w_panel = wp;
  return launched(q8::launch_gemm(q8::GEMM_INT8_DECOMP, g, Q8_F16, st));
}

q8_status q8_linear_fp8(const void* x, int64_t M, int64_t K, const uint8_t* wq, const float* w_scale,
                        int64_t N, float scale_ub, const float* bias, void* y, void* workspace,
                        size_t workspace_bytes, void* stream) {
  Q8_TRY(check_mnk(M, N, K));
  if (!wq || !w_scale || (M > 0 && (!x || !y))) return Q8_ERR_NULL_PTR;
  if (std::isnan(scale_ub) || scale_ub <= 0.0f) return Q8_ERR_BAD_ARG;
  const Fp8Ws ws = fp8_ws(M, K);
  if (ws.total > 0 && (!workspace || workspace_bytes < ws.total)) return Q8_ERR_WORKSPACE;
  if (!aligned16(x) || !aligned16(wq) || !aligned16(w_scale) || !aligned16(y) || !aligned16(workspace) ||
      (bias && !aligned16(bias)))
    return Q8_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Q8_TRY(check_device(st));
  Q8_TRY(check_ptrs(st, {x, wq, w_scale, bias, y, workspace}));
  if (M == 0) return Q8_OK;

  char* base = static_cast<char*>(workspace);
  uint8_t* xq = reinterpret_cast<uint8_t*>(base + ws.xq);
  float* xs = reinterpret_cast<float*>(base + ws.xs);
  Q8_TRY(launched(q8::launch_quant_rows_fp8(x, Q8_BF16, M, K, scale_ub, xq, xs, st)));
  q8::GemmArgs g{};
  g.a = xq;
  g.b = wq;
  g.a_scale = xs;
  g.b_scale = w_scale;
  g.bias = bias;
  g.y = y;
  g.M = M;
  g.N = N;
  g.K = K;
  return launched(q8::launch_gemm(q8::GEMM_FP8, g, Q8_BF16, st));
}

q8_status q8_linear_fp8_grouped(const void* x, int64_t T, int64_t K, const int32_t* expert_offsets, int64_t E,
                                const uint8_t* wq, const float* w_scale, int64_t N, float scale_ub, void* y,
                                void* workspace, size_t workspace_bytes, void* stream) {
  Q8_TRY(check_mnk(T, N, K));
  if (E < 1 || E > kMaxGroups || E * N > kMaxRows) return Q8_ERR_BAD_SHAPE;
  if (!expert_offsets || !wq || !w_scale || (T > 0 && (!x || !y))) return Q8_ERR_NULL_PTR;
  if (std::isnan(scale_ub) || scale_ub <= 0.0f) return Q8_ERR_BAD_ARG;
  const Fp8Ws ws = fp8_ws(T, K);
  if (ws.total > 0 && (!workspace || workspace_bytes < ws.total)) return Q8_ERR_WORKSPACE;
  if (!aligned16(x) || !aligned16(wq) || !aligned16(w_scale) || !aligned16(y) || !aligned16(workspace) ||
      !aligned4(expert_offsets))
    return Q8_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Q8_TRY(check_device(st));
  Q8_TRY(check_ptrs(st, {x, expert_offsets, wq, w_scale, y, workspace}));
  if (T == 0) return Q8_OK;

  char* base = static_cast<char*>(workspace);
  uint8_t* xq = reinterpret_cast<uint8_t*>(base + ws.xq);
  float* xs = reinterpret_cast<float*>(base + ws.xs);
  // per-token scales do not depend on the expert: one pass over all routed rows
  Q8_TRY(launched(q8::launch_quant_rows_fp8(x, Q8_BF16, T, K, scale_ub, xq, xs, st)));
  q8::GemmArgs g{};
  g.a = xq;
  g.b = wq;
  g.a_scale = xs;
  g.b_scale = w_scale;
  g.y = y;
  g.M = T;
  g.N = N;
  g.K = K;
  g.groups = (int)E;
  g.group_offsets = expert_offsets;
  return launched(q8::launch_gemm_fp8_grouped(g, st));
}

q8_status q8_gemm_int8(const int8_t* xq, const float* x_scale, const int32_t* x_rowsum, int64_t M,
                       int64_t K, const int8_t* wq, const float* w_scale, const float* w_zp, int64_t N,
                       const float* bias, void* y, q8_dtype y_dtype, int32_t* acc_out, void* stream) {
  if (!valid_dtype(y_dtype)) return Q8_ERR_BAD_DTYPE;
  Q8_TRY(check_mnk(M, N, K));
  if (!wq || !w_scale || !w_zp || (M > 0 && (!xq || !x_scale || !x_rowsum || !y))) return Q8_ERR_NULL_PTR;
  if (!aligned16(xq) || !aligned16(x_scale) || !aligned16(x_rowsum) || !aligned16(wq) ||
      !aligned16(w_scale) || !aligned16(w_zp) || !aligned16(y) || (bias && !aligned16(bias)) ||
      (acc_out && !aligned16(acc_out)))
    return Q8_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Q8_TRY(check_device(st));
  Q8_TRY(check_ptrs(st, {xq, x_scale, x_rowsum, wq, w_scale, w_zp, bias, y, acc_out}));
  if (M == 0) return Q8_OK;
  return launched(int8_on_codes(xq, x_scale, x_rowsum, M, K, wq, w_scale, w_zp, N, bias, y, y_dtype, acc_out, st));
}

q8_status q8_quantize_act_static(const void* x, q8_dtype x_dtype, int64_t M, int64_t K, float x_scale,
                                 int8_t* xq, int32_t* x_rowsum, void* stream) {
  if (!valid_dtype(x_dtype)) return Q8_ERR_BAD_DTYPE;
  Q8_TRY(check_mk(M, K, 0));
  if (M > 0 && (!x || !xq)) return Q8_ERR_NULL_PTR;
  if (!std::isfinite(x_scale) || x_scale <= 0.0f) return Q8_ERR_BAD_ARG;
  if (!aligned16(x) || !aligned16(xq) || (x_rowsum && !aligned16(x_rowsum))) return Q8_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Q8_TRY(check_device(st));
  Q8_TRY(check_ptrs(st, {x, xq, x_rowsum}));
  if (M == 0) return Q8_OK;
  return launched(q8::launch_quant_act_i8_static(x, x_dtype, M, K, x_scale, xq, nullptr, x_rowsum, st));
}

q8_status q8_linear_static(const void* x, q8_dtype x_dtype, int64_t M, int64_t K, float x_scale,
                           const int8_t* wq, const float* w_scale, const float* w_zp, int64_t N,
                           const float* bias, float y_scale, int8_t* yq, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (!valid_dtype(x_dtype)) return Q8_ERR_BAD_DTYPE;
  Q8_TRY(check_mnk(M, N, K));
  if (!wq || !w_scale || !w_zp || (M > 0 && (!x || !yq))) return Q8_ERR_NULL_PTR;
  if (!std::isfinite(x_scale) || x_scale <= 0.0f || !std::isfinite(y_scale) || y_scale <= 0.0f)
    return Q8_ERR_BAD_ARG;
  const LinearWs ws = static_ws(M, K);
  if (ws.total > 0 && (!workspace || workspace_bytes < ws.total)) return Q8_ERR_WORKSPACE;
  if (!aligned16(x) || !aligned16(wq) || !aligned16(w_scale) || !aligned16(w_zp) || !aligned16(yq) ||
      (bias && !aligned16(bias)) || !aligned16(workspace))
    return Q8_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Q8_TRY(check_device(st));
  Q8_TRY(check_ptrs(st, {x, wq, w_scale, w_zp, bias, yq, workspace}));
  if (M == 0) return Q8_OK;
  char* base = static_cast<char*>(workspace);
  int8_t* xq = reinterpret_cast<int8_t*>(base + ws.xq);
  float* xs = reinterpret_cast<float*>(base + ws.xs);
  int32_t* rs = reinterpret_cast<int32_t*>(base + ws.rs);
  Q8_TRY(launched(q8::launch_quant_act_i8_static(x, x_dtype, M, K, x_scale, xq, xs, rs, st)));
  const double y_inv = 1.0 / (double)y_scale;
  return launched(int8_on_codes(xq, xs, rs, M, K, wq, w_scale, w_zp, N, bias, yq, q8::kOutInt8, nullptr, st, y_inv));
}

q8_status q8_linear_w8a16(const void* x, q8_dtype x_dtype, int64_t M, int64_t K, const int8_t* wq,
                          const float* w_scale, const float* w_zp, int64_t N, const float* bias, void* y,
                          q8_dtype y_dtype, void* stream) {
  if (!valid_dtype(x_dtype) || !valid_dtype(y_dtype) || x_dtype == Q8_F32) return Q8_ERR_BAD_DTYPE;
  Q8_TRY(check_mnk(M, N, K));
  if (M > q8::kW8A16MaxM) return Q8_ERR_BAD_SHAPE;
  if (!wq || !w_scale || !w_zp || (M > 0 && (!x || !y))) return Q8_ERR_NULL_PTR;
  if (!aligned16(x) || !aligned16(wq) || !aligned16(w_scale) || !aligned16(w_zp) || !aligned16(y) ||
      (bias && !aligned16(bias)))
    return Q8_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Q8_TRY(check_device(st));
  Q8_TRY(check_ptrs(st, {x, wq, w_scale, w_zp, bias, y}));
  if (M == 0) return Q8_OK;
  return launched(q8::launch_gemv_w8a16(x, x_dtype, M, K, wq, w_scale, w_zp, N, bias, y, y_dtype, st));
}

q8_status q8_quantize_weight_grouped(const void* w, q8_dtype w_dtype, int64_t N, int64_t K, int64_t group,
                                     int8_t* wq, float* w_scale, float* w_zp, void* stream) {
  if (!valid_dtype(w_dtype)) return Q8_ERR_BAD_DTYPE;
  Q8_TRY(check_mk(N, K));
  if (!valid_group(group, K)) return Q8_ERR_BAD_SHAPE;
  if (!w || !wq || !w_scale || !w_zp) return Q8_ERR_NULL_PTR;
  if (!aligned16(w) || !aligned16(wq) || !aligned16(w_scale) || !aligned16(w_zp)) return Q8_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Q8_TRY(check_device(st));
  Q8_TRY(check_ptrs(st, {w, wq, w_scale, w_zp}));
  return launched(q8::launch_quant_weight_grouped(w, w_dtype, N, K, group, wq, w_scale, w_zp, st));
}

q8_status q8_linear_grouped(const void* x, q8_dtype x_dtype, int64_t M, int64_t K, const int8_t* wq,
                            const float* w_scale, const float* w_zp, int64_t group, int64_t N, const float* bias,
                            void* y, q8_dtype y_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_dtype(x_dtype) || !valid_dtype(y_dtype)) return Q8_ERR_BAD_DTYPE;
  Q8_TRY(check_mnk(M, N, K));
  if (!valid_group(group, K)) return Q8_ERR_BAD_SHAPE;
  if (!wq || !w_scale || !w_zp || (M > 0 && (!x || !y))) return Q8_ERR_NULL_PTR;
  const GroupedWs ws = grouped_ws(M, K);
  if (ws.total > 0 && (!workspace || workspace_bytes < ws.total)) return Q8_ERR_WORKSPACE;
  if (!aligned16(x) || !aligned16(wq) || !aligned16(w_scale) || !aligned16(w_zp) || !aligned16(y) ||
      (bias && !aligned16(bias)) || (ws.total > 0 && !aligned16(workspace)))
    return Q8_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Q8_TRY(check_device(st));
  Q8_TRY(check_ptrs(st, {x, wq, w_scale, w_zp, bias, y, workspace}));
  if (M == 0) return Q8_OK;
  if (M <= q8::kGemvFusedMaxM)
    return launched(q8::launch_gemv_i8_grouped(x, x_dtype, M, K, wq, w_scale, w_zp, group, N, bias, y, y_dtype, st));
  char* base = static_cast<char*>(workspace);
  int8_t* xq = reinterpret_cast<int8_t*>(base + ws.xq);
  float* xs = reinterpret_cast<float*>(base + ws.xs);
  int32_t* gs = reinterpret_cast<int32_t*>(base + ws.gs);
  Q8_TRY(launched(q8::launch_quant_act_i8_groups(x, x_dtype, M, K, group, xq, xs, gs, st)));
  if (M <= q8::kGroupGemvMaxM)
    return launched(q8::launch_gemv_group(xq, xs, gs, M, K, wq, w_scale, w_zp, group, N, bias, y, y_dtype, st));
  return launched(q8::launch_gemm_group(xq, xs, gs, M, K, wq, w_scale, w_zp, group, N, bias, y, y_dtype, st));
}

q8_status q8_bench_mfma_loop(q8_format fmt, int64_t iters, int64_t workgroups, int32_t* sink, void* stream) {
  if (fmt != Q8_INT8_SYM && fmt != Q8_FP8_E4M3) return Q8_ERR_BAD_FORMAT;
  if (iters < 1 || iters > kMaxRows || workgroups < 1 || workgroups > 65536) return Q8_ERR_BAD_ARG;
  if (!sink) return Q8_ERR_NULL_PTR;
  if (!aligned16(sink)) return Q8_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Q8_TRY(check_device(st));
  Q8_TRY(check_ptrs(st, {sink}));
  return launched(q8::launch_mfma_loop(fmt == Q8_INT8_SYM ? 0 : 2, iters, workgroups, sink, st));
}

q8_status q8_bench_stream_read(const void* src, int64_t bytes, int64_t workgroups, int32_t* sink, void* stream) {
  if (bytes < 16 || bytes % 16 != 0 || bytes >= (int64_t(1) << 31) || workgroups < 1 || workgroups > 65536)
    return Q8_ERR_BAD_ARG;
  if (!src || !sink) return Q8_ERR_NULL_PTR;
  if (!aligned16(src) || !aligned16(sink)) return Q8_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Q8_TRY(check_device(st));
  Q8_TRY(check_ptrs(st, {src, sink}));
  return launched(q8::launch_stream_read(src, bytes, workgroups, sink, st));
}

q8_status q8_probe_fp8_mfma(const uint8_t* a, const uint8_t* b, const float* c, float* d, int64_t count,
                            void* stream) {
  if (count < 1 || count > 65536) return Q8_ERR_BAD_ARG;
  if (!a || !b || !c || !d) return Q8_ERR_NULL_PTR;
  if (!aligned16(a) || !aligned16(b) || !aligned16(c) || !aligned16(d)) return Q8_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Q8_TRY(check_device(st));
  Q8_TRY(check_ptrs(st, {a, b, c, d}));
  return launched(q8::launch_probe_fp8_mfma(a, b, c, d, count, st));
}

q8_status q8_gemm_tile(q8_op op, int64_t M, int64_t N, int64_t K, int32_t* bm, int32_t* bn) {
  if (op != Q8_OP_LINEAR && op != Q8_OP_STATIC && op != Q8_OP_DECOMP && op != Q8_OP_FP8) return Q8_ERR_BAD_ARG;
  Q8_TRY(check_mnk(M, N, K));
  if (!bm || !bn) return Q8_ERR_NULL_PTR;
  *bm = *bn = 0;
  if (M == 0 || ((op == Q8_OP_LINEAR || op == Q8_OP_STATIC) && M <= q8::kGemvMaxM)) return Q8_OK;
  const q8::GemmKind kind = op == Q8_OP_DECOMP ? q8::GEMM_INT8_DECOMP : op == Q8_OP_FP8 ? q8::GEMM_FP8 : q8::GEMM_INT8;
  int tm = 0, tn = 0;
  q8::gemm_tile(kind, M, N, &tm, &tn);
  *bm = tm;
  *bn = tn;
  return Q8_OK;
}

q8_status q8_gemm_fp8(const uint8_t* xq, const float* x_scale, int64_t M, int64_t K, const uint8_t* wq,
                      const float* w_scale, int64_t N, const float* bias, void* y, void* stream) {
  Q8_TRY(check_mnk(M, N, K));
  if (!wq || !w_scale || (M > 0 && (!xq || !x_scale || !y))) return Q8_ERR_NULL_PTR;
  if (!aligned16(xq) || !aligned16(x_scale) || !aligned16(wq) || !aligned16(w_scale) || !aligned16(y) ||
      (bias && !aligned16(bias)))
    return Q8_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Q8_TRY(check_device(st));
  Q8_TRY(check_ptrs(st, {xq, x_scale, wq, w_scale, bias, y}));
  if (M == 0) return Q8_OK;
  q8::GemmArgs g{};
  g.a = xq;
  g.b = wq;
  g.a_scale = x_scale;
  g.b_scale = w_scale;
  g.bias = bias;
  g.y = y;
  g.M = M;
  g.N = N;
  g.K = K;
  return launched(q8::launch_gemm(q8::GEMM_FP8, g, Q8_BF16, st));
}

}  // extern "C"
