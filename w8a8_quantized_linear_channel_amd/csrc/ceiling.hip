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

// One FP8 MFMA per wave on operands from memory.  Lane l supplies row l % 32
// of both operands, bytes 32 (l / 32) .. +31 of its 64 (the mapping the GEMM's
// fragments use); output register r of lane l is row 8 (r / 4) + 4 (l / 32) +
// r % 4, column l % 32 (the 32 x 32 MFMA output layout).
__global__ __launch_bounds__(64) void k_probe_fp8(const uint8_t* __restrict__ a, const uint8_t* __restrict__ b,
                                                  const float* __restrict__ c, float* __restrict__ d) {
  const int lane = threadIdx.x, p = blockIdx.x;
  const int row = lane & 31, kh = lane >> 5;
  const v4i* pa = (const v4i*)(a + (size_t)p * 2048 + row * 64 + kh * 32);
  const v4i* pb = (const v4i*)(b + (size_t)p * 2048 + row * 64 + kh * 32);
  const v4i a0 = pa[0], a1 = pa[1], b0 = pb[0], b1 = pb[1];
  const v8i fa = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
  const v8i fb = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
  v16f acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = 8 * (r >> 2) + 4 * kh + (r & 3);
    acc[r] = c[(size_t)p * 1024 + i * 32 + row];
  }
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb, acc, 0, 0, 0, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = 8 * (r >> 2) + 4 * kh + (r & 3);
    d[(size_t)p * 1024 + i * 32 + row] = acc[r];
  }
}

// Streaming read: every thread reads 16-byte chunks of [src, src + bytes) at
// a grid stride, eight loads in flight, with the non-temporal cache policy the
// decode kernels use for their weights; the chunks are xor-folded into one
// word per thread.
__global__ __launch_bounds__(256) void k_stream_read(const uint8_t* __restrict__ src, uint32_t chunks,
                                                     int* __restrict__ sink) {
  const uint32_t stride = gridDim.x * blockDim.x;
  uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  const __amdgpu_buffer_rsrc_t r = byte_buffer(src, chunks * 16u);
  v4i acc = {0, 0, 0, 0};
  for (; i + 7 * stride < chunks; i += 8 * stride) {
    v4i v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = load16_nt(r, (i + u * stride) * 16u);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u];
  }
  for (; i < chunks; i += stride) acc ^= load16_nt(r, i * 16u);
  sink[blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace

hipError_t launch_stream_read(const void* src, int64_t bytes, int64_t workgroups, int* sink, hipStream_t st) {
  k_stream_read<<<(unsigned)workgroups, 256, 0, st>>>((const uint8_t*)src, (uint32_t)(bytes / 16), sink);
  return hipGetLastError();
}

hipError_t launch_probe_fp8_mfma(const uint8_t* a, const uint8_t* b, const float* c, float* d, int64_t count,
                                 hipStream_t st) {
  k_probe_fp8<<<(unsigned)count, 64, 0, st>>>(a, b, c, d);
  return hipGetLastError();
}

hipError_t launch_mfma_loop(int kind, int64_t iters, int64_t workgroups, int* sink, hipStream_t st) {
  if (kind == 0) k_mfma_loop<0><<<(unsigned)workgroups, 256, 0, st>>>((int)iters, sink);
  else k_mfma_loop<2><<<(unsigned)workgroups, 256, 0, st>>>((int)iters, sink);
  return hipGetLastError();
}

}  // namespace q8
