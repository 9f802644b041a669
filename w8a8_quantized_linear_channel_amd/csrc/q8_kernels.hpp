// Internal launchers of the libq8 kernels (host side, not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8 {

// Quantizers (quant.hip); dt / ydt use the q8_dtype numbering.
hipError_t launch_quant_weight_i8(const void* w, int dt, int64_t N, int64_t K, int8_t* wq,
                                  float* w_scale, float* w_zp, hipStream_t st);
hipError_t launch_quant_rows_fp8(const void* x, int dt, int64_t R, int64_t K, float bound,
                                 uint8_t* xq, float* x_scale, hipStream_t st);
// Static INT8 activation codes with a given per-tensor scale (quant.hip);
// x_scale (nullable) receives the scale on every row.
hipError_t launch_quant_act_i8_static(const void* x, int dt, int64_t M, int64_t K, float scale, int8_t* xq,
                                      float* x_scale, int32_t* x_rowsum, hipStream_t st);
hipError_t launch_quant_act_i8(const void* x, int dt, int64_t M, int64_t K, int8_t* xq, float* x_scale,
                               int32_t* x_rowsum, hipStream_t st);
// LLM.int8: the first kPanelCols outlier columns in compact form for the
// GEMM's outlier flow, row-major with kPanelCols fp16 values per row and
// zeros past the outlier count: x_panel [M] rows hold X[m, O_j], w_panel [N]
// rows hold fp16(fp32(S_w[n] (wq[n, O_j] - Z_w[n]))).
constexpr int kPanelCols = 16;
struct OutlierPanels {
  const int8_t* wq;         // [N, K] weight codes
  const float* w_scale;     // [N]
  const float* w_zp;        // [N]
  int64_t N;
  uint16_t* x_panel;        // [M, kPanelCols] or null (no panels)
  uint16_t* w_panel;        // [N, kPanelCols]
};
// fp16 activations of the LLM.int8 step: columns with flags[k] != 0 read as 0
// (flags may be null: none); also writes the ascending outlier list idx[] and
// its count cnt[0] (and copies to user_idx / user_cnt when not null), and the
// panels when p.x_panel is not null.
hipError_t launch_quant_act_f16_outliers(const uint16_t* x, int64_t M, int64_t K, const uint8_t* flags,
                                         int8_t* xq, float* x_scale, int32_t* x_rowsum, int32_t* idx,
                                         int32_t* cnt, int32_t* user_idx, int32_t* user_cnt,
                                         const OutlierPanels& p, hipStream_t st);

// Operands and epilogue inputs of the MFMA GEMM (gemm.hip).
struct GemmArgs {
  const uint8_t* a;         // [M, K] activation codes (int8 or e4m3 bytes)
  const uint8_t* b;         // [N, K] weight codes
  const float* a_scale;     // [M]
  const int32_t* a_rowsum;  // [M], int8 paths
  const float* b_scale;     // [N]
  const float* b_zp;        // [N], int8 paths
  const float* bias;        // [N] or null
  void* y;                  // [M, N] of ydt
  int32_t* acc_out;         // [M, N] or null (int8 paths)
  int64_t M, N, K;
  // LLM.int8 outlier flow
  const uint16_t* x_f16;    // [M, K] fp16 activations
  const int32_t* out_idx;   // ascending outlier columns
  const int32_t* out_cnt;   // [1] number of outlier columns (device)
  const uint16_t* x_panel;  // [M, kPanelCols] the first outlier columns of X (fp16)
  const uint16_t* w_panel;  // [N, kPanelCols] their fp16 weights
  // INT8 output (ydt DT_I8): 1 / S_y of the static output scale
  double y_inv;
  // grouped problems (experts): groups > 0 and the device row offsets [groups+1]
  int groups;
  const int32_t* group_offsets;
};

// Output dtype code of the requantized INT8 output (the device enum's DT_I8;
// q8_dtype has F32 = 0, F16 = 1, BF16 = 2).
constexpr int kOutInt8 = 3;

enum GemmKind : int { GEMM_INT8 = 0, GEMM_INT8_DECOMP = 1, GEMM_FP8 = 2 };

hipError_t launch_gemm(GemmKind kind, const GemmArgs& g, int ydt, hipStream_t st);
// The output tile (BM x BN) launch_gemm uses for an M x N problem of `kind`.
void gemm_tile(GemmKind kind, int64_t M, int64_t N, int* bm, int* bn);
// FP8 rowwise GEMM over groups of rows (bf16 out): g.M is the total row count,
// g.b / g.b_scale hold groups consecutive [N, K] / [N] blocks.
hipError_t launch_gemm_fp8_grouped(const GemmArgs& g, hipStream_t st);

// Decode-shaped int8 linear (gemv.hip).  M <= kGemvFusedMaxM: one launch with
// the activation quantization fused in; kGemvFusedMaxM < M <= kGemvMaxM: on
// codes, scales and code sums from the row quantizer.
hipError_t launch_gemv_i8(const void* x, int xdt, int64_t M, int64_t K, const int8_t* wq,
                          const float* w_scale, const float* w_zp, int64_t N, const float* bias,
                          void* y, int ydt, int32_t* acc_out, hipStream_t st);
hipError_t launch_gemv_q8(const int8_t* xq, const float* x_scale, const int32_t* x_rowsum, int64_t M, int64_t K,
                          const int8_t* wq, const float* w_scale, const float* w_zp, int64_t N, const float* bias,
                          void* y, int ydt, int32_t* acc_out, hipStream_t st, double y_inv = 0.0);
constexpr int64_t kGemvFusedMaxM = 10;

// Weight-only W8A16 linear for decode-sized M (w8a16.hip): x bf16 or f16.
hipError_t launch_gemv_w8a16(const void* x, int xdt, int64_t M, int64_t K, const int8_t* wq, const float* w_scale,
                             const float* w_zp, int64_t N, const float* bias, void* y, int ydt, hipStream_t st);
constexpr int64_t kW8A16MaxM = 16;
constexpr int64_t kGemvMaxM = 16;

// LLM.int8 outlier columns (decomp.hip): flags[k] = max_m |x[m,k]| >= threshold
// (threshold > 0).
hipError_t launch_outlier_flags(const uint16_t* x_f16, int64_t M, int64_t K, float threshold, uint8_t* flags,
                                hipStream_t st);

}  // namespace q8
