/*
 * Measurement helper of libq8, outside the quantized layer itself: a
 * register-only MFMA loop that gives the matrix-core rate the chip sustains
 * with no memory traffic (the measured compute ceiling set beside the
 * published peak when the GEMM kernels are timed).
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

#ifdef __cplusplus
}
#endif

#endif /* Q8_BENCH_H */
