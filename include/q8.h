/*
 * q8.h -- C ABI of libq8, the 8-bit quantized linear layer Y = X . W^T on one
 * AMD Instinct MI355X (gfx950).
 *
 * Pages cited (by title and section):
 *   [LF]   "8-Bit LLM Quantization with Lightning Fabric"
 *   [OV]   "大模型量化技术概述" (LLM quantization overview, devpress)
 *   [FB]   "Transformers FP8 (W8A8) 量化实战：基于 FBGEMM 的模型压缩与加载"
 *   [BNB]  "Transformers 单 GPU 高效推理：bitsandbytes LLM.int8 8-bit 混合精度量化的原理与实操"
 *   [NOTE] Xilyfe, "大模型量化" (lecture notes)
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every tensor pointer is DEVICE memory owned by the caller.  The library
 *   never allocates, frees or keeps a pointer after a call returns.  Scratch
 *   space comes from a caller-provided workspace sized by q8_workspace_bytes
 *   (q8_linear_noalloc: from a fixed device array of the library).
 * - Tensors are dense, row-major, 2-D.  X is [M, K] (tokens x input features),
 *   W is [N, K] (output features x input features, K contiguous), Y is [M, N].
 *   A caller with batch dimensions flattens them into M first ([FB] §5.2: the
 *   input is viewed as 2-D) and reshapes Y back afterwards.
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *   Calls only enqueue work on that stream and return; no call ever waits for
 *   the device, so results are valid once the stream has reached this point.
 *   The library keeps no state between calls apart from a per-device cache of
 *   the device check (and the scratch array of q8_linear_noalloc); calls on
 *   different streams may run concurrently (q8_linear_noalloc excepted).
 * - Every argument is checked on the host BEFORE anything is enqueued.  On a
 *   non-Q8_OK status nothing has been written.  Q8_ERR_LAUNCH reports a
 *   failed kernel launch (hipGetLastError) after validation passed.
 * - Empty batches: every call that takes activations accepts M = 0 (T = 0
 *   for q8_linear_fp8_grouped).  It checks its other arguments as usual; the
 *   pointers to M-sized arrays (x, codes, scales, code sums, y, acc_out) may
 *   then be NULL, no workspace is needed (q8_workspace_bytes returns 0), and
 *   nothing is enqueued or written, except that q8_linear_int8_decomp writes
 *   0 to n_outliers when it is given (the outlier set of no rows is empty).
 * - Preconditions checked for every call: M >= 0 and N, K >= 1 (weight
 *   quantization: N, K >= 1); K % 16 == 0;
 *   K <= 65536 (keeps the zero-point-corrected INT32 sums in range); every
 *   matrix (X, W, Y) has fewer than 2^31 elements; all pointers 16-byte
 *   aligned; the device running `stream` is gfx950.
 *   Inputs must be finite: NaN/Inf inputs give unspecified codes and outputs.
 * - Floating point follows IEEE binary32 with round-to-nearest-even; scales
 *   are computed with correctly rounded division, codes with x / S (not
 *   x * (1/S)); nothing is flushed to zero.
 */
#ifndef Q8_H
#define Q8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum q8_status {
  Q8_OK = 0,
  Q8_ERR_NULL_PTR = 1,   /* a required pointer is NULL */
  Q8_ERR_BAD_SHAPE = 2,  /* M < 0, N or K < 1, K % 16 != 0, or a size overflows */
  Q8_ERR_BAD_DTYPE = 3,  /* unsupported element type for this argument */
  Q8_ERR_BAD_FORMAT = 4, /* unsupported quantization format for this call */
  Q8_ERR_BAD_ARG = 5,    /* NaN threshold/bound, or a pointer that must be NULL is not */
  Q8_ERR_ALIGN = 6,      /* a pointer is not 16-byte aligned */
  Q8_ERR_WORKSPACE = 7,  /* workspace NULL or smaller than q8_workspace_bytes */
  Q8_ERR_DEVICE = 8,     /* no HIP device, or the device is not gfx950 */
  Q8_ERR_LAUNCH = 9      /* a kernel launch failed */
} q8_status;

typedef enum q8_dtype { Q8_F32 = 0, Q8_F16 = 1, Q8_BF16 = 2 } q8_dtype;

typedef enum q8_format {
  Q8_INT8_ASYM = 0, /* weights: per-row asymmetric int8, r = S (q - Z)         */
  Q8_INT8_SYM = 1,  /* activations: per-row symmetric int8, r = S q           */
  Q8_FP8_E4M3 = 2   /* weights or activations: per-row OCP e4m3fn, r = S q    */
} q8_format;

typedef enum q8_op {
  Q8_OP_LINEAR = 0, Q8_OP_DECOMP = 1, Q8_OP_FP8 = 2, Q8_OP_STATIC = 3, Q8_OP_GROUPED = 4
} q8_op;

/*
 * q8_quantize_weight -- per-output-channel weight quantization (done once,
 * off the per-token path).
 *
 * Q8_INT8_ASYM  ([LF] §2.1 per-channel asymmetric scale and zero-point, §3.3
 *   quantizer; [OV] §2.3 min-max S = (R_max - R_min)/(Q_max - Q_min),
 *   Z = Q_min - round(R_min/S); [NOTE] "量化是什么" r = S (q - Z)).  Per row n:
 *     lo = min(0, min_k w), hi = max(0, max_k w)
 *     S  = max((hi - lo) / 255, 1e-8)
 *     Z  = -128 - rne(lo / S)                         (integer in [-128, 127])
 *     q  = clamp(rne(w / S) + Z, -128, 127)
 *   wq: int8 [N, K]; w_scale: float [N]; w_zp: float [N] holding the integer Z.
 * Q8_FP8_E4M3  ([FB] §5.1: e4m3fn weight, one fp32 weight_scale per output
 *   channel).  Per row n: S = max(max_k |w| / 448, 1e-8),
 *   q = e4m3_rne(clamp(w / S, -448, 448)).  wq: uint8 e4m3fn codes [N, K];
 *   w_scale: float [N]; w_zp must be NULL (else Q8_ERR_BAD_ARG).
 * w: [N, K] of type w_dtype (F32, F16 or BF16).
 * Errors: Q8_ERR_BAD_FORMAT for fmt == Q8_INT8_SYM.
 */
q8_status q8_quantize_weight(q8_format fmt, const void* w, q8_dtype w_dtype,
                             int64_t N, int64_t K, void* wq, float* w_scale,
                             float* w_zp, void* stream);

/*
 * q8_quantize_act -- dynamic per-token activation quantization (recomputed at
 * every forward: [NOTE] dynamic quantization section; [FB] §5.2).
 *
 * Q8_INT8_SYM  ([NOTE] symmetric section and QuantInt8 code).  Per row m:
 *     S = max(max_k |x| / 127, 1e-8);  q = clamp(rne(x / S), -127, 127)
 *   xq: int8 [M, K]; x_scale: float [M]; x_rowsum: int32 [M] = sum_k q (the
 *   term the weight zero-point correction needs), may be NULL.  scale_ub is
 *   ignored.
 * Q8_FP8_E4M3  ([FB] §1, §4, §6: per-row e4m3 with the activation scale upper
 *   bound, default 1200).  Per row m:
 *     a = min(max_k |x|, scale_ub);  S = max(a / 448, 1e-8)
 *     q = e4m3_rne(clamp(x / S, -448, 448))
 *   scale_ub = +INFINITY means no bound; NaN or <= 0 is Q8_ERR_BAD_ARG.
 *   xq: uint8 e4m3fn codes [M, K]; x_scale: float [M]; x_rowsum must be NULL.
 * x: [M, K] of type x_dtype (F32, F16 or BF16).
 * Errors: Q8_ERR_BAD_FORMAT for fmt == Q8_INT8_ASYM.
 */
q8_status q8_quantize_act(q8_format fmt, const void* x, q8_dtype x_dtype,
                          int64_t M, int64_t K, float scale_ub, void* xq,
                          float* x_scale, int32_t* x_rowsum, void* stream);

/*
 * q8_linear -- W8A8 linear layer: dynamic per-token INT8 X, per-channel
 * asymmetric INT8 W, INT8 x INT8 products with INT32 accumulation ([NOTE]
 * "INT8 这么小的范围不会导致溢出吗？"), then the dequantization epilogue
 * ([OV] §2.1 quantized matmul, read as Y = S_x X_q . (S_w (W_q - Z_w))^T):
 *     acc[m,n] = sum_k xq[m,k] wq[n,k]                      (exact int32)
 *     y[m,n]   = S_x[m] S_w[n] (acc[m,n] - Z_w[n] sum_k xq[m,k]) (+ bias[n])
 * The activation quantization is the Q8_INT8_SYM rule above.  For M <= 10 it
 * is fused into the one kernel; for larger M the codes, scales and code sums
 * pass through the workspace (for M <= 16 into a streaming GEMV, above into
 * the MFMA GEMM).
 * x: [M, K] of x_dtype (F32, F16, BF16); wq/w_scale/w_zp: from
 * q8_quantize_weight(Q8_INT8_ASYM); bias: float [N] or NULL; y: [M, N] of
 * y_dtype (F32, F16, BF16).  acc_out: int32 [M, N] debug copy of acc, or NULL.
 * workspace: q8_workspace_bytes(Q8_OP_LINEAR, M, N, K) bytes (0 for M <= 10).
 */
q8_status q8_linear(const void* x, q8_dtype x_dtype, int64_t M, int64_t K,
                    const int8_t* wq, const float* w_scale, const float* w_zp,
                    int64_t N, const float* bias, void* y, q8_dtype y_dtype,
                    void* workspace, size_t workspace_bytes, int32_t* acc_out,
                    void* stream);

/*
 * q8_linear_int8_decomp -- LLM.int8() mixed-precision decomposition ([BNB]
 * core idea: outlier feature columns go through a 16-bit product, the regular
 * ~99.9% of values through int8; BitsAndBytesConfig table: threshold 6.0,
 * 0.0 maximizes the int8 share).
 *     O = { k : max_m |x[m,k]| >= threshold }  (ascending; empty if threshold <= 0)
 *     X_R = X with the columns O set to 0, quantized as Q8_INT8_SYM (so the
 *           per-token scale is taken over the regular columns only)
 *     W_O[n,j] = fp16(S_w[n] (wq[n,O_j] - Z_w[n]))    (no fp16 weight copy kept)
 *     y = [int8 path of q8_linear on X_R] + X[:,O] . W_O^T (+ bias)
 * x: fp16 [M, K]; y: fp16 [M, N]; weights as for q8_linear.
 * outlier_idx: int32 [K] receives O in ascending order (entries past the
 * count are unspecified), or NULL; n_outliers: int32 [1] receives |O|, or
 * NULL.  Both stay on the device: the call never synchronizes.
 * acc_out: int32 [M, N] debug copy of the int8-path accumulator, or NULL.
 * threshold NaN is Q8_ERR_BAD_ARG.
 * workspace: q8_workspace_bytes(Q8_OP_DECOMP, M, N, K) bytes: the activation
 * codes, scales and row sums, the column flags, the outlier list and count,
 * and the first 16 outlier columns of X and of W_O in compact fp16 form
 * ((M + N) x 32 bytes), which the product reads instead of gathering them.
 */
q8_status q8_linear_int8_decomp(const void* x, int64_t M, int64_t K,
                                const int8_t* wq, const float* w_scale,
                                const float* w_zp, int64_t N, float threshold,
                                const float* bias, void* y, void* workspace,
                                size_t workspace_bytes, int32_t* outlier_idx,
                                int32_t* n_outliers, int32_t* acc_out,
                                void* stream);

/*
 * q8_linear_fp8 -- FP8 e4m3 W8A8 rowwise linear ([FB] §5.2 per-row dynamic
 * activation quantization with the scale upper bound; §5.3 fp8 x fp8 product
 * with row scales on both sides, bf16 output, fp32 bias added after):
 *     xq, S_x = Q8_FP8_E4M3 activation rule with scale_ub
 *     y[m,n]  = (sum_k e4m3(xq[m,k]) e4m3(wq[n,k]))  S_x[m] S_w[n] (+ bias[n])
 * Products are exact; the sum is accumulated in fp32.
 * x: bf16 [M, K] (other dtypes are Q8_ERR_BAD_DTYPE: the page's forward is
 * bf16 only); wq: e4m3fn codes [N, K] and w_scale float [N] from
 * q8_quantize_weight(Q8_FP8_E4M3); bias: float [N] or NULL; y: bf16 [M, N].
 * scale_ub as for q8_quantize_act.  workspace: q8_workspace_bytes(Q8_OP_FP8).
 */
q8_status q8_linear_fp8(const void* x, int64_t M, int64_t K, const uint8_t* wq,
                        const float* w_scale, int64_t N, float scale_ub,
                        const float* bias, void* y, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * q8_gemm_int8 -- the INT8 GEMM and dequantization epilogue of q8_linear on
 * activations that are already quantized (by q8_quantize_act(Q8_INT8_SYM), or
 * shared by several projections of the same X):
 *     acc[m,n] = sum_k xq[m,k] wq[n,k];  y = S_x[m] S_w[n] (acc - Z_w[n] x_rowsum[m]) (+ bias)
 * ([NOTE] "INT8 这么小的范围不会导致溢出吗？": INT32 accumulation; [OV] §2.1
 * quantized matmul with r = S (q - Z)).  xq: int8 [M, K]; x_scale: float [M];
 * x_rowsum: int32 [M] (= sum_k xq, required); weights, bias, y, y_dtype and
 * acc_out as for q8_linear.  No workspace.  q8_linear with M > 10 is exactly
 * q8_quantize_act followed by this call.
 */
q8_status q8_gemm_int8(const int8_t* xq, const float* x_scale, const int32_t* x_rowsum,
                       int64_t M, int64_t K, const int8_t* wq, const float* w_scale,
                       const float* w_zp, int64_t N, const float* bias, void* y,
                       q8_dtype y_dtype, int32_t* acc_out, void* stream);

/*
 * q8_gemm_fp8 -- the rowwise FP8 product on quantized operands, the shape of
 * the page's f8f8bf16_rowwise(xq, w, x_scale, w_scale) ([FB] §5.3):
 *     y[m,n] = (sum_k e4m3(xq[m,k]) e4m3(wq[n,k])) S_x[m] S_w[n] (+ bias[n])
 * xq: e4m3fn codes [M, K] with x_scale float [M] (from q8_quantize_act
 * (Q8_FP8_E4M3)); wq, w_scale, bias as for q8_linear_fp8; y: bf16 [M, N].
 * No workspace.  q8_linear_fp8 is q8_quantize_act followed by this call.
 */
q8_status q8_gemm_fp8(const uint8_t* xq, const float* x_scale, int64_t M, int64_t K,
                      const uint8_t* wq, const float* w_scale, int64_t N, const float* bias,
                      void* y, void* stream);

/*
 * q8_linear_fp8_grouped -- FP8 expert projection of a mixture-of-experts layer
 * on routed tokens ([FB] §5.4, Llama4 experts: per-expert FP8 weights with
 * per-row scales; each expert's tokens get per-token FP8 quantization and the
 * rowwise FP8 product with that expert's weights).  Rows
 * expert_offsets[e] .. expert_offsets[e+1]-1 of x belong to expert e:
 *     y[t,n] = S_x[t] S_w[e,n] sum_k e4m3(xq[t,k]) e4m3(wq[e,n,k])   (fp32 acc)
 * with the activation quantization of q8_quantize_act(Q8_FP8_E4M3, scale_ub).
 * x: bf16 [T, K] grouped by expert; expert_offsets: int32 [E+1] in DEVICE
 * memory, non-decreasing from 0 to T (the offsets are read on the device and
 * never copied to the host; values outside [0, T] or decreasing are clamped,
 * which may leave rows of y unwritten but never reads or writes outside the
 * arrays); wq: e4m3 [E, N, K] and w_scale: float [E, N] from
 * q8_quantize_weight(Q8_FP8_E4M3) on the [E*N, K] view; y: bf16 [T, N].
 * workspace: q8_workspace_bytes(Q8_OP_FP8, T, N, K).  Errors: Q8_ERR_BAD_SHAPE
 * unless 1 <= E <= 1024; Q8_ERR_BAD_ARG for a NaN or non-positive scale_ub.
 */
q8_status q8_linear_fp8_grouped(const void* x_bf16, int64_t T, int64_t K,
                                const int32_t* expert_offsets, int64_t E,
                                const uint8_t* wq, const float* w_scale, int64_t N,
                                float scale_ub, void* y_bf16, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * q8_quantize_act_static -- static INT8 activation quantization ("lecture
 * notes on LLM quantization", static quantization: the scale is calibrated
 * beforehand and applied unchanged at inference): one float scale S for the
 * tensor, xq = clamp(rne(x / S), -127, 127) with the binary32 division,
 * x_rowsum[m] = sum_k xq[m,k] (nullable).  x: [M, K] of x_dtype; xq: int8
 * [M, K].  Errors: Q8_ERR_BAD_ARG unless 0 < x_scale < inf.
 */
q8_status q8_quantize_act_static(const void* x, q8_dtype x_dtype, int64_t M, int64_t K,
                                 float x_scale, int8_t* xq, int32_t* x_rowsum, void* stream);

/*
 * q8_linear_static -- W8A8 linear with a static activation scale and an INT8
 * output for the next layer (same notes, "INT8 这么小的范围不会导致溢出吗？", step 4:
 * the INT32 result is scaled back into INT8):
 *     xq = q8_quantize_act_static(x, x_scale);  acc = sum_k xq wq  (exact int32)
 *     v  = (x_scale S_w[n]) (acc - Z_w[n] sum_k xq) (+ bias[n])       (float64)
 *     yq = clamp(rne(v * (1 / y_scale)), -127, 127)                   (float64)
 * x: [M, K] of x_dtype; weights from q8_quantize_weight(Q8_INT8_ASYM); bias:
 * float [N] or NULL; yq: int8 [M, N].  workspace:
 * q8_workspace_bytes(Q8_OP_STATIC, M, N, K) bytes.  Errors: Q8_ERR_BAD_ARG
 * unless both scales are finite and positive.
 */
q8_status q8_linear_static(const void* x, q8_dtype x_dtype, int64_t M, int64_t K, float x_scale,
                           const int8_t* wq, const float* w_scale, const float* w_zp, int64_t N,
                           const float* bias, float y_scale, int8_t* yq, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * q8_linear_w8a16 -- weight-only linear for decode-sized M: the INT8
 * asymmetric weights are dequantized for a product with the 16-bit
 * activations, which are not quantized ("lecture notes on LLM quantization",
 * PTQ section, weight quantization):
 *     y[m,n] = S_w[n] Sum_k x[m,k] (wq[n,k] - Z_w[n])  (+ bias[n])
 * The widened weights are exact; products accumulate in fp32.
 * x: [M, K] of x_dtype (BF16 or F16 only); wq/w_scale/w_zp: from
 * q8_quantize_weight(Q8_INT8_ASYM); bias: float [N] or NULL; y: [M, N] of
 * y_dtype (F32, F16, BF16).  No workspace.
 * Errors: Q8_ERR_BAD_DTYPE for an F32 x; Q8_ERR_BAD_SHAPE for M > 16, besides
 * the preconditions above.
 */
q8_status q8_linear_w8a16(const void* x, q8_dtype x_dtype, int64_t M, int64_t K,
                          const int8_t* wq, const float* w_scale, const float* w_zp,
                          int64_t N, const float* bias, void* y, q8_dtype y_dtype,
                          void* stream);

/*
 * q8_quantize_weight_grouped -- per-group asymmetric INT8 weights ("大模型量化
 * 技术概述" §2.2, granularity: groups of 64 to 128 parameters, each with its
 * own parameters; lecture notes' granularity passage: per-group blocks with
 * their own scale and zero point).  Group j of row n is w[n, j g .. j g + g-1];
 * each group is quantized as Q8_INT8_ASYM quantizes a row:
 *     lo = min(0, min w), hi = max(0, max w), S = max((hi - lo)/255, 1e-8),
 *     Z = -128 - rne(lo / S),  q = clamp(rne(w / S) + Z, -128, 127)
 * w: [N, K] of w_dtype; group: 64 or 128 and K a multiple of it (else
 * Q8_ERR_BAD_SHAPE); wq: int8 [N, K]; w_scale, w_zp: float [K/group, N],
 * group-major (w_scale[j * N + n] belongs to group j of row n; w_zp holds the
 * integer Z).
 */
q8_status q8_quantize_weight_grouped(const void* w, q8_dtype w_dtype, int64_t N, int64_t K,
                                     int64_t group, int8_t* wq, float* w_scale, float* w_zp,
                                     void* stream);

/*
 * q8_linear_grouped -- W8A8 linear with per-group weights: the activations are
 * quantized per token as q8_quantize_act(Q8_INT8_SYM) does, and the
 * quantized-matmul identity is taken group by group ([OV] §2.1 with r = S (q - Z)):
 *     C_j[m,n] = sum_{k in j} xq[m,k] wq[n,k] - Z[j,n] sum_{k in j} xq[m,k]   (exact)
 *     y[m,n]   = S_x[m] sum_j S[j,n] C_j[m,n]  (+ bias[n])                    (fp32)
 * x: [M, K] of x_dtype; wq/w_scale/w_zp from q8_quantize_weight_grouped with
 * the same group; bias: float [N] or NULL; y: [M, N] of y_dtype.  workspace:
 * q8_workspace_bytes(Q8_OP_GROUPED, M, N, K) bytes: none up to 10 tokens
 * (the quantization is fused into the decode kernel), else codes, scales and
 * group code sums, sized for group 64.  Errors: Q8_ERR_BAD_SHAPE for a group
 * other than 64 or 128 or a K that is not a multiple of it.
 */
q8_status q8_linear_grouped(const void* x, q8_dtype x_dtype, int64_t M, int64_t K,
                            const int8_t* wq, const float* w_scale, const float* w_zp,
                            int64_t group, int64_t N, const float* bias, void* y,
                            q8_dtype y_dtype, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * q8_linear_noalloc -- q8_linear with no workspace argument, for callers that
 * cannot allocate device memory around a call (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Same arguments,
 * computation, kernels and results as q8_linear, bit for bit.  The scratch
 * that q8_linear takes from the workspace (above 10 tokens: the activation
 * codes, scales and code sums, q8_workspace_bytes(Q8_OP_LINEAR, M, N, K)
 * bytes) comes from a library-owned 32 MiB device array per GPU, created with
 * the library and kept until the process ends; nothing is allocated or freed
 * by the call.  Every call on one GPU shares that GPU's array: calls that may
 * overlap on one GPU (other streams, other host threads) race and must be
 * ordered by the caller.  The array keeps the last call's contents; nothing
 * in it needs to start at zero.  The first call on a device looks up the
 * array's address there (host side, once per device).
 * Errors: as q8_linear, and Q8_ERR_WORKSPACE if the scratch the shape needs
 * exceeds 32 MiB (M * K + 8 M plus alignment: e.g. M = 4096 at K = 8192).
 */
q8_status q8_linear_noalloc(const void* x, q8_dtype x_dtype, int64_t M, int64_t K,
                            const int8_t* wq, const float* w_scale, const float* w_zp,
                            int64_t N, const float* bias, void* y, q8_dtype y_dtype,
                            int32_t* acc_out, void* stream);

/* Bytes of workspace the call `op` needs at this shape (0 if none); returns 0
 * for invalid shapes as well, which the call itself then rejects. */
size_t q8_workspace_bytes(q8_op op, int64_t M, int64_t N, int64_t K);

/* Static, human-readable name of a status code. */
const char* q8_status_str(q8_status s);

#ifdef __cplusplus
}
#endif

#endif /* Q8_H */
