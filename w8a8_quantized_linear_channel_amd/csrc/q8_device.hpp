// Device-side helpers shared by the libq8 kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8 {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// Element types of X / W / Y, matching q8_dtype.
enum Dt : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_I8 = 3 /* requantized INT8 output (internal) */ };

constexpr float kEps = 1e-8f;        // floor of every scale
constexpr float kFp8Max = 448.0f;    // largest finite OCP e4m3fn value

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Decode one 16-byte chunk of a row into floats: 4 for fp32, 8 for fp16/bf16.
template <int DT> struct Chunk;
template <> struct Chunk<DT_F32> {
  static constexpr int kElems = 4;
  __device__ __forceinline__ static void decode(const v4i& c, float* v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __int_as_float(c[i]);
  }
};
template <> struct Chunk<DT_F16> {
  static constexpr int kElems = 8;
  __device__ __forceinline__ static void decode(const v4i& c, float* v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t u = (uint32_t)c[i];
      v[2 * i] = f16_bits_to_f32(u & 0xffffu);
      v[2 * i + 1] = f16_bits_to_f32(u >> 16);
    }
  }
};
template <> struct Chunk<DT_BF16> {
  static constexpr int kElems = 8;
  __device__ __forceinline__ static void decode(const v4i& c, float* v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t u = (uint32_t)c[i];
      v[2 * i] = __uint_as_float(u << 16);
      v[2 * i + 1] = __uint_as_float(u & 0xffff0000u);
    }
  }
};

// fp32 -> bf16 / fp16 with round-to-nearest-even (hardware conversions).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Two outputs packed into one word, round-to-nearest-even: one
// v_cvt_pk_bf16_f32 for bf16.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
template <int DT> __device__ __forceinline__ uint32_t pack2_out(float a, float b);
template <> __device__ __forceinline__ uint32_t pack2_out<DT_BF16>(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), bf16x2_t));
}
template <> __device__ __forceinline__ uint32_t pack2_out<DT_F16>(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), f16x2_t));
}

template <int DT> __device__ __forceinline__ void store_out(void* y, int64_t i, float v);
template <> __device__ __forceinline__ void store_out<DT_F32>(void* y, int64_t i, float v) {
  ((float*)y)[i] = v;
}
template <> __device__ __forceinline__ void store_out<DT_F16>(void* y, int64_t i, float v) {
  ((uint16_t*)y)[i] = f32_to_f16(v);
}
template <> __device__ __forceinline__ void store_out<DT_BF16>(void* y, int64_t i, float v) {
  ((uint16_t*)y)[i] = f32_to_bf16(v);
}

// Wave64 reductions (butterfly over all 64 lanes).
// Wave-wide reductions; every lane gets the result.  Four DPP steps reduce
// each row of 16 lanes (quad_perm [1,0,3,2] and [2,3,0,1] pair lanes within a
// quad, row_half_mirror pairs the two quads of each half-row, row_mirror the
// two halves of the row); the four row results are then read as scalars.
// DPP moves run in the VALU, unlike a ds_bpermute butterfly whose six steps
// each wait on the LDS crossbar.
template <typename Op>
__device__ __forceinline__ int dpp_row_reduce(int v, Op op) {
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false));
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false));
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  const int r = dpp_row_reduce(__float_as_int(v), [](int a, int b) {
    return __float_as_int(fmaxf(__int_as_float(a), __int_as_float(b)));
  });
  const float a = __int_as_float(__builtin_amdgcn_readlane(r, 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(r, 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(r, 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(r, 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}
__device__ __forceinline__ float wave_min(float v) {
  const int r = dpp_row_reduce(__float_as_int(v), [](int a, int b) {
    return __float_as_int(fminf(__int_as_float(a), __int_as_float(b)));
  });
  const float a = __int_as_float(__builtin_amdgcn_readlane(r, 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(r, 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(r, 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(r, 48));
  return fminf(fminf(a, b), fminf(c, d));
}
// Inclusive prefix sum over the 64 lanes of a wave (all lanes active): row
// shifts by 1, 2, 4 and 8 inside each 16-lane row, then lane 15's total of
// rows 0 and 2 into rows 1 and 3, then lane 31's total of rows 0-1 into rows
// 2 and 3.  Lanes with no source lane keep the 0 passed as the old value.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31 into rows 2, 3
  return v;
}
__device__ __forceinline__ int wave_sum(int v) {
  const int r = dpp_row_reduce(v, [](int a, int b) { return a + b; });
  return __builtin_amdgcn_readlane(r, 0) + __builtin_amdgcn_readlane(r, 16) +
         __builtin_amdgcn_readlane(r, 32) + __builtin_amdgcn_readlane(r, 48);
}

// Block-wide reductions for blocks of NW waves; `red` is LDS of >= NW slots.
// Every thread gets the result.
template <int NW>
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = fmaxf(r, red[i]);
  return r;
}
template <int NW>
__device__ __forceinline__ float block_min(float v, float* red) {
  v = wave_min(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = fminf(r, red[i]);
  return r;
}
template <int NW>
__device__ __forceinline__ int block_sum(int v, int* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  int r = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) r += red[i];
  return r;
}

// The quotient x / s rounded to binary32, from r = RN(1/s) with two FMAs
// (y0 = x r, e = x - s y0 exactly, y1 = y0 + e r).  Used for 16-bit inputs with
// a scale derived from the row absmax: over that whole domain the int8 and
// e4m3 codes taken from y1 equal those of the correctly rounded quotient
// (verified exhaustively on the host for every bf16 / fp16 x and absmax).
__device__ __forceinline__ float quot_fma(float x, float s, float r) {
#pragma clang fp contract(off)
  const float y0 = x * r;
  const float e = __builtin_fmaf(-s, y0, x);
  return __builtin_fmaf(e, r, y0);
}

// Round-to-nearest-even to an integer by adding 1.5 * 2^23: for |y| < 2^22 the
// low byte of the sum's bit pattern is rne(y) as a two's-complement int8.
__device__ __forceinline__ uint32_t rne_int8_bits(float y) {
#pragma clang fp contract(off)
  return __float_as_uint(y + 12582912.0f);
}

// Low bytes of four words, packed little-endian into one word (v_perm_b32).
__device__ __forceinline__ uint32_t pack_lo_bytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);
  const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x0c0c0400u);
  return __builtin_amdgcn_perm(cd, ab, 0x05040100u);
}

// Sum of the four signed bytes of a packed word, added to acc (v_dot4_i32_i8).
__device__ __forceinline__ int sum_i8x4(uint32_t packed, int acc) {
  return __builtin_amdgcn_sdot4((int)packed, 0x01010101, acc, false);
}

// Symmetric int8 code: clamp(rne(x / s), -127, 127) with IEEE division.
__device__ __forceinline__ int code_sym_i8(float x, float s) {
  float q = __builtin_rintf(x / s);
  q = fminf(fmaxf(q, -127.0f), 127.0f);
  return (int)q;
}

// Four e4m3fn codes (ties to even) of values already clamped to [-448, 448],
// packed little-endian into one word.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  int p = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  p = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, p, true);
  return (uint32_t)p;
}

// Outlier weight of the LLM.int8 flow: fp16(fp32(S (q - Z))), the product
// rounded to fp32 before the conversion to fp16, as the dequantized fp32
// weights are cast to fp16.  Left alone, the compiler fuses the multiply and
// the conversion into one v_fma_mixlo_f16 (even with contraction off), which
// rounds the exact product to fp16 once and differs from the two roundings
// next to a tie of fp16; the empty asm makes the fp32 product a value of its
// own.
__device__ __forceinline__ _Float16 outlier_weight_f16(float s, int q, float z) {
  float p = s * ((float)q - z);
  asm volatile("" : "+v"(p));
  return (_Float16)p;
}

__device__ __forceinline__ uint32_t pack4_i8(int a, int b, int c, int d) {
  return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
         ((uint32_t)(d & 0xff) << 24);
}

// s_waitcnt immediate for lgkmcnt(0) alone on gfx9: vmcnt 63 (bits 3:0 and
// 15:14), expcnt 7 (bits 6:4), lgkmcnt 0 (bits 11:8)
constexpr int kLgkmcnt0 = 0xC07F;

typedef __attribute__((address_space(3))) void* lptr_t;   // LDS

// global_load_lds_dwordx4: 64 lanes x 16 bytes from gbase + voff (per lane)
// into 1 KB of LDS at `lds` (lane l at lds + 16 l), counted by vmcnt.  Issued
// as inline asm on purpose: the compiler's own wait insertion cannot tell the
// LDS a DMA fills from the LDS other reads come from and would put a
// vmcnt(0) before every LDS read, draining any prefetch.  Callers wait for
// the DMA themselves (s_waitcnt vmcnt, plus a barrier when other waves read
// the data).  M0 carries the LDS address; nothing else in these kernels uses
// M0, and the s_nop covers the M0-write -> LDS-DMA hazard.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// INT8 requantized output: clamp(rne(((S_x S_w) C + b) / S_y), +-127) with the
// division as the product by inv = 1 / S_y, every step in float64 and none
// contracted, so the code is decided exactly as the definition states.
__device__ __forceinline__ int requant_i8(float sx, float sw, int c, float b, double inv) {
#pragma clang fp contract(off)
  double v = ((double)sx * (double)sw) * (double)c;
  v = v + (double)b;
  // the clamp as one float64 max and min (for finite values the same as the
  // compare-and-select form, which takes six 32-bit instructions)
  const double q = __builtin_fmin(__builtin_fmax(rint(v * inv), -127.0), 127.0);
  return (int)q;
}

// A buffer resource for raw byte loads over [p, p + bytes) (word 3 for raw
// byte access on gfx9): loads past the end return zeros instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t byte_buffer(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
// 16 bytes at byte offset off with the non-temporal cache policy (streamed once)
__device__ __forceinline__ v4i load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}

__device__ __forceinline__ void dma16(const uint8_t* gbase, uint32_t voff, uint8_t* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(lptr_t)lds;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(m0), "v"(voff), "s"(gbase)
               : "memory", "m0");
}
// As dma16, from a per-lane 64-bit address.
__device__ __forceinline__ void dma16_ptr(const void* gp, uint8_t* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(lptr_t)lds;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(m0), "v"(gp)
               : "memory", "m0");
}
#pragma clang diagnostic pop

}  // namespace q8
