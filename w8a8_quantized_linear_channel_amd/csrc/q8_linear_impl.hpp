// q8_linear split in two (api.cpp), shared by q8_linear and the
// allocation-free q8_linear_noalloc (noalloc.hip).  Host side only.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "q8.h"

namespace q8 {

// The checks of q8_linear that need no device (dtypes, shapes, pointers,
// alignment); *workspace_needed receives q8_workspace_bytes(Q8_OP_LINEAR).
q8_status linear_check_args(const void* x, q8_dtype x_dtype, int64_t M, int64_t K, const int8_t* wq,
                            const float* w_scale, const float* w_zp, int64_t N, const float* bias, const void* y,
                            q8_dtype y_dtype, const int32_t* acc_out, size_t* workspace_needed);
// The rest of q8_linear: device check, then the launches, with `workspace`
// (16-byte aligned, at least workspace_needed bytes) as scratch.
q8_status linear_run(const void* x, q8_dtype x_dtype, int64_t M, int64_t K, const int8_t* wq, const float* w_scale,
                     const float* w_zp, int64_t N, const float* bias, void* y, q8_dtype y_dtype, void* workspace,
                     int32_t* acc_out, void* stream);
// The device that runs `stream` (the current device for NULL).
q8_status stream_device(void* stream, int* dev);

}  // namespace q8
