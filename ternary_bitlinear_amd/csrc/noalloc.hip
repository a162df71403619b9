// bitlinear_forward_f32 for callers that cannot allocate: the workspace comes
// from a fixed array in device memory that the library owns, not from the
// caller.
//
// The array is a file-scope __device__ variable, so each GPU the library runs
// on holds its own copy, reserved when the library's code is loaded on that
// device and kept until the process ends.  In host code its name is only a
// stand-in for the symbol: its device address comes from hipGetSymbolAddress,
// resolved once per device (with that device current) on the first call there
// and kept per device.  Kernels receive that address, never the name.
//
// Every call on one GPU shares that GPU's array; the kernels need no part of
// it cleared (every byte they read was written earlier in the same call), so
// nothing is reset between calls, and two calls that overlap in time on one
// GPU (different streams, or host threads) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/bitlinear.h"
#include "kernels.hpp"

namespace {

constexpr size_t kScratchBytes = (size_t)BITLINEAR_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// The device address of this device's scratch array (resolved on first use).
hipError_t scratch_ptr(int dev, void** out) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

namespace bl {

size_t noalloc_scratch_bytes() { return kScratchBytes; }

// Arguments are validated by the caller (the ABI layer), which also checked
// that the workspace the call needs fits kScratchBytes.
hipError_t launch_forward_f32_noalloc(const uint8_t* W_packed, const float* gamma, int64_t N,
                                      int64_t K, const float* X, int64_t M, void* Y, int y_dtype,
                                      int8_t* X_q_out, float* x_scale_out, int32_t* x_sum_out,
                                      hipStream_t stream) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* ws = nullptr;
  e = scratch_ptr(dev, &ws);
  if (e != hipSuccess) return e;
  return launch_forward_f32(W_packed, gamma, N, K, X, nullptr, M, Y, y_dtype, X_q_out,
                            x_scale_out, x_sum_out, ws, stream);
}

}  // namespace bl
