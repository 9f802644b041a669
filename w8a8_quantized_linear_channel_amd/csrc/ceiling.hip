// Register-only MFMA loops: the matrix-core rate the chip sustains with no
// memory traffic at all, the measured compute ceiling that the GEMM kernels
// are set beside (next to the published peak).  Each wave runs `iters`
// rounds of four independent MFMAs on operands held in registers; one value
// per lane is stored at the end so that nothing is optimized away.
#include "q8_device.hpp"
#include "q8_bench_kernels.hpp"

namespace q8 {
namespace {

template <int KIND>   // 0: v_mfma_i32_32x32x32_i8, 2: v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3)
__global__ __launch_bounds__(256) void k_mfma_loop(int iters, int* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  int s = 0;
  if constexpr (KIND == 0) {
    const v4i a = {lane * 3 + 1, lane ^ 0x5a5a5a5a, lane * 7, 0x01020304 + lane};
    const v4i b = {0x11223344 - lane, lane * 5 + 2, lane ^ 0x0f0f0f0f, lane * 11};
    v16i c0{}, c1{}, c2{}, c3{};
    for (int i = 0; i < iters; ++i) {
      c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, b, c3, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c0[r] ^ c1[r] ^ c2[r] ^ c3[r];
  } else {
    // e4m3 bytes 0x38 (1.0) and 0x30 (0.5) mixed with the lane: finite codes
    const int pa = 0x38383838 ^ (lane & 0x03030303), pb = 0x30303030 ^ ((lane >> 2) & 0x03030303);
    const v8i a = {pa, pb, pa, pb, pa, pb, pa, pb}, b = {pb, pa, pb, pa, pb, pa, pb, pa};
    v16f c0{}, c1{}, c2{}, c3{};
    for (int i = 0; i < iters; ++i) {
      c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 0, 0, 0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c1, 0, 0, 0, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, c2, 0, 0, 0, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, b, c3, 0, 0, 0, 0, 0, 0);
    }
    float t = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) t += c0[r] + c1[r] + c2[r] + c3[r];
    s = __float_as_int(t);
  }
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_mfma_loop(int kind, int64_t iters, int64_t workgroups, int* sink, hipStream_t st) {
  if (kind == 0) k_mfma_loop<0><<<(unsigned)workgroups, 256, 0, st>>>((int)iters, sink);
  else k_mfma_loop<2><<<(unsigned)workgroups, 256, 0, st>>>((int)iters, sink);
  return hipGetLastError();
}

}  // namespace q8
