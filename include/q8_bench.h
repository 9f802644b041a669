/*
 * Measurement helpers of libq8, outside the quantized layer itself:
 * - a register-only MFMA loop that gives the matrix-core rate the chip
 *   sustains with no memory traffic (the measured compute ceiling set beside
 *   the published peak when the GEMM kernels are timed);
 * - a streaming read of a device buffer, the measured HBM ceiling set beside
 *   the published bandwidth when the HBM-bound kernels are timed;
 * - a probe that runs the FP8 GEMM's matrix instruction once on given
 *   operands, so that the rounding of its internal sum can be measured
 *   against exact sums (the FP8 parity tolerance rests on it);
 * - a query of the GEMM tile a call picks for a shape, so that tests can
 *   show which kernel instantiation a shape exercises.
 */
#ifndef Q8_BENCH_H
#define Q8_BENCH_H

#include "q8.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * q8_bench_mfma_loop -- launches `workgroups` workgroups of 256 threads (four
 * waves); every wave runs `iters` rounds of four independent MFMAs on
 * register operands and each thread writes one int to sink.
 *   fmt Q8_INT8_SYM:  v_mfma_i32_32x32x32_i8, 65536 int8 ops per MFMA
 *   fmt Q8_FP8_E4M3:  v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3), 131072 flops per MFMA
 * Ops per launch: workgroups * 4 waves * iters * 4 MFMAs * (ops per MFMA).
 * sink: device int32 [workgroups * 256], caller-owned.  Asynchronous on
 * `stream`.  Errors: Q8_ERR_BAD_FORMAT for other formats; Q8_ERR_BAD_ARG
 * unless 1 <= iters < 2^31 and 1 <= workgroups <= 65536; Q8_ERR_NULL_PTR,
 * Q8_ERR_ALIGN (sink 16-byte aligned), Q8_ERR_DEVICE as for every call.
 */
q8_status q8_bench_mfma_loop(q8_format fmt, int64_t iters, int64_t workgroups, int32_t* sink,
                             void* stream);

/*
 * q8_bench_stream_read -- reads `bytes` of device memory at `src` once:
 * `workgroups` x 256 threads, each reading 16-byte chunks at a grid stride
 * with eight loads in flight and the non-temporal cache policy of the
 * decode kernels' weight stream, xor-folding them into sink[t] (device int32
 * [workgroups * 256], caller-owned).  Asynchronous on `stream`.
 * Errors: Q8_ERR_BAD_ARG unless bytes is a positive multiple of 16 below
 * 2^31 and 1 <= workgroups <= 65536; Q8_ERR_NULL_PTR, Q8_ERR_ALIGN (src and
 * sink 16-byte aligned), Q8_ERR_DEVICE as for every call.
 */
q8_status q8_bench_stream_read(const void* src, int64_t bytes, int64_t workgroups, int32_t* sink,
                               void* stream);

/*
 * q8_probe_fp8_mfma -- for each of `count` independent problems p, one wave
 * runs one v_mfma_f32_32x32x64_f8f6f4 on e4m3 operands (the instruction and
 * operand layout of the FP8 GEMM's main loop: the scaled form with zero scale
 * operands, which the compiler emits as this unscaled instruction)
 *     d[p][i][j] = c[p][i][j] + sum_{k<64} e4m3(a[p][i][k]) e4m3(b[p][j][k])
 * a, b: uint8 e4m3fn codes [count, 32, 64] (row-major, k contiguous); c, d:
 * float [count, 32, 32] (row-major).  The page's FP8 GEMM runs with fast
 * accumulation ("Transformers FP8 (W8A8) 量化实战…" §5.3,
 * use_fast_accum=True): the instruction's own sum is not exact, and this
 * probe is how its error is measured.  Device memory, caller-owned, 16-byte
 * aligned; asynchronous on `stream`.  Errors: Q8_ERR_BAD_ARG unless
 * 1 <= count <= 65536; Q8_ERR_NULL_PTR, Q8_ERR_ALIGN, Q8_ERR_DEVICE as for
 * every call.
 */
q8_status q8_probe_fp8_mfma(const uint8_t* a, const uint8_t* b, const float* c, float* d,
                            int64_t count, void* stream);

/*
 * q8_gemm_tile -- the output tile (rows x columns of Y per workgroup) of the
 * MFMA GEMM that a call of `op` runs for M activation rows and N output
 * features: *bm x *bn is 256 x 256, 128 x 128, 64 x 128 or 64 x 64.  Writes
 * 0 x 0 where no GEMM runs (Q8_OP_LINEAR and Q8_OP_STATIC up to 16 rows,
 * which take the streaming decode kernels, and M = 0).  Q8_OP_LINEAR is
 * q8_linear / q8_gemm_int8, Q8_OP_STATIC q8_linear_static, Q8_OP_DECOMP
 * q8_linear_int8_decomp, Q8_OP_FP8 q8_linear_fp8 / q8_gemm_fp8.  Host only,
 * nothing is launched.  Errors: Q8_ERR_BAD_ARG for another op;
 * Q8_ERR_BAD_SHAPE for shapes the calls reject; Q8_ERR_NULL_PTR.
 */
q8_status q8_gemm_tile(q8_op op, int64_t M, int64_t N, int64_t K, int32_t* bm, int32_t* bn);

#ifdef __cplusplus
}
#endif

#endif /* Q8_BENCH_H */
