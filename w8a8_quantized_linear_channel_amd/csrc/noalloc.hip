// q8_linear_noalloc: q8_linear without a caller workspace, for callers that
// cannot allocate (code under HIP graph capture, tight serving loops).  Its
// scratch (the activation codes, scales and code sums that pass between the
// row quantizer and the GEMM above 10 tokens) lives in one file-scope device
// array of kScratchBytes per GPU, kept until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: the
// device address of each GPU's copy is taken once per device with
// hipGetSymbolAddress (that device current) and only that address is passed
// to the kernels.  Nothing here allocates.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "q8.h"
#include "q8_linear_impl.hpp"

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;   // 32 MiB per GPU
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of `scratch` on device `dev`, looked up on the first
// call for that device and kept.
q8_status scratch_on(int dev, void** out) {
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      int cur = -1;
      if (hipGetDevice(&cur) != hipSuccess) {
        (void)hipGetLastError();
        return Q8_ERR_DEVICE;
      }
      if (cur != dev && hipSetDevice(dev) != hipSuccess) {
        (void)hipGetLastError();
        return Q8_ERR_DEVICE;
      }
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (cur != dev) (void)hipSetDevice(cur);
      if (e != hipSuccess || p == nullptr) {
        (void)hipGetLastError();
        return Q8_ERR_DEVICE;
      }
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return Q8_OK;
}

}  // namespace

extern "C" q8_status q8_linear_noalloc(const void* x, q8_dtype x_dtype, int64_t M, int64_t K, const int8_t* wq,
                                       const float* w_scale, const float* w_zp, int64_t N, const float* bias,
                                       void* y, q8_dtype y_dtype, int32_t* acc_out, void* stream) {
  size_t need = 0;
  q8_status s = q8::linear_check_args(x, x_dtype, M, K, wq, w_scale, w_zp, N, bias, y, y_dtype, acc_out, &need);
  if (s != Q8_OK) return s;
  if (need > kScratchBytes) return Q8_ERR_WORKSPACE;
  int dev = -1;
  s = q8::stream_device(stream, &dev);
  if (s != Q8_OK) {
    (void)hipGetLastError();
    return s;
  }
  if (dev < 0 || dev >= kMaxDevices) return Q8_ERR_DEVICE;
  void* ptr = nullptr;
  s = scratch_on(dev, &ptr);
  if (s != Q8_OK) return s;
  return q8::linear_run(x, x_dtype, M, K, wq, w_scale, w_zp, N, bias, y, y_dtype, ptr, acc_out, stream);
}
