// Host-side check of the C ABI's argument validation, built with address and
// undefined-behaviour sanitizers on the host code (device code unchanged).
// Every call here is rejected before any HIP call, or (when no GPU is
// visible) reaches the device check and reports BITLINEAR_ERR_NO_DEVICE; no
// kernel is ever launched.  Prints "abi_check ok" and returns 0 on success.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/bitlinear.h"

static int failures = 0;

// value check without the last-error requirement (size and kernel queries)
static void expect_value(const char* what, long long got, long long want) {
  if (got != want) {
    std::printf("FAIL %s: %lld, want %lld\n", what, got, want);
    ++failures;
  }
}

static void expect(const char* what, int got, int want) {
  if (got != want) {
    std::printf("FAIL %s: status %d, want %d (%s)\n", what, got, want, bitlinear_last_error());
    ++failures;
  } else if (want != BITLINEAR_OK && std::strlen(bitlinear_last_error()) == 0) {
    std::printf("FAIL %s: no error message\n", what);
    ++failures;
  }
}

int main() {
  int ndev = 0;
  const bool no_gpu = hipGetDeviceCount(&ndev) != hipSuccess || ndev == 0;
  // aligned placeholder addresses, never dereferenced
  void* P = reinterpret_cast<void*>(uintptr_t(1) << 20);
  void* U = reinterpret_cast<void*>((uintptr_t(1) << 20) + 2);   // misaligned
  const uint8_t* W = static_cast<const uint8_t*>(P);
  const float* F = static_cast<const float*>(P);
  const int8_t* Q = static_cast<const int8_t*>(P);
  const int32_t* S = static_cast<const int32_t*>(P);
  const int64_t M = 2, N = 64, K = 128;

  // size queries on invalid and boundary shapes
  expect_value("packed_bytes K%16", (int)bitlinear_packed_bytes(4, 40), 0);
  expect_value("packed_bytes K max+16", (int)bitlinear_packed_bytes(4, BITLINEAR_MAX_K + 16), 0);
  expect_value("pack ws N*K>=2^31", (int)bitlinear_pack_workspace_bytes(int64_t(1) << 20, 1 << 12), 0);
  expect_value("forward ws M=0", (int)bitlinear_forward_workspace_bytes(0, N, K), 0);
  expect_value("forward ws N huge", (int)bitlinear_forward_workspace_bytes(M, int64_t(1) << 40, K), 0);
  expect_value("grouped ws G=0", (int)bitlinear_forward_grouped_workspace_bytes(M, 0, &N, K), 0);
  expect_value("grouped ws null N", (int)bitlinear_forward_grouped_workspace_bytes(M, 2, nullptr, K), 0);
  expect_value("kernel query bad entry", bitlinear_forward_kernel(7, M, 1, &N, K), -BITLINEAR_ERR_SHAPE);
  expect_value("kernel query null N", bitlinear_forward_kernel(0, M, 1, nullptr, K), -BITLINEAR_ERR_SHAPE);

  // each validation status of each entry point
  expect("pack null", bitlinear_pack_weights(nullptr, N, K, (uint8_t*)P, (float*)P, P, 1 << 20, nullptr),
         BITLINEAR_ERR_NULL);
  expect("pack shape", bitlinear_pack_weights(F, N, 40, (uint8_t*)P, (float*)P, P, 1 << 20, nullptr),
         BITLINEAR_ERR_SHAPE);
  expect("pack align", bitlinear_pack_weights((const float*)U, N, K, (uint8_t*)P, (float*)P, P, 1 << 20, nullptr),
         BITLINEAR_ERR_ALIGN);
  expect("pack workspace", bitlinear_pack_weights(F, N, K, (uint8_t*)P, (float*)P, P, 8, nullptr),
         BITLINEAR_ERR_WORKSPACE);
  expect("quant null", bitlinear_quant_acts(F, M, K, nullptr, (float*)P, (int32_t*)P, nullptr),
         BITLINEAR_ERR_NULL);
  expect("quant shape", bitlinear_quant_acts(F, 0, K, (int8_t*)P, (float*)P, (int32_t*)P, nullptr),
         BITLINEAR_ERR_SHAPE);
  expect("quant bits", bitlinear_quant_acts_bits(F, M, K, 3, (int8_t*)P, (float*)P, (int32_t*)P, nullptr),
         BITLINEAR_ERR_DTYPE);
  expect("forward dtype", bitlinear_forward(W, F, N, K, Q, F, S, M, P, (bitlinear_dtype)9, P, 1 << 20, nullptr),
         BITLINEAR_ERR_DTYPE);
  expect("forward align Y", bitlinear_forward(W, F, N, K, Q, F, S, M, U, BITLINEAR_F32, P, 1 << 20, nullptr),
         BITLINEAR_ERR_ALIGN);
  expect("forward shape K", bitlinear_forward(W, F, N, BITLINEAR_MAX_K + 16, Q, F, S, M, P, BITLINEAR_F32, P,
                                              1 << 20, nullptr),
         BITLINEAR_ERR_SHAPE);
  expect("forward workspace", bitlinear_forward(W, F, 8192, 12288, Q, F, S, 64, P, BITLINEAR_BF16, nullptr, 0,
                                                nullptr),
         BITLINEAR_ERR_WORKSPACE);
  expect("forward_f32 outputs", bitlinear_forward_f32(W, F, N, K, F, M, P, BITLINEAR_F32, (int8_t*)P, nullptr,
                                                      nullptr, P, 1 << 20, nullptr),
         BITLINEAR_ERR_NULL);
  expect("noalloc too big", bitlinear_forward_f32_noalloc(W, F, 256, 32768, F, 2048, P, BITLINEAR_BF16, nullptr,
                                                          nullptr, nullptr, nullptr),
         BITLINEAR_ERR_WORKSPACE);
  expect("rmsnorm null gain", bitlinear_rmsnorm_quant(F, nullptr, M, K, (int8_t*)P, (float*)P, (int32_t*)P,
                                                      nullptr),
         BITLINEAR_ERR_NULL);
  const uint8_t* Ws[5] = {W, W, W, W, W};
  const float* Gs[5] = {F, F, F, F, F};
  void* Ys[5] = {P, P, P, P, P};
  const int64_t Ns[5] = {N, N, N, N, N};
  expect("grouped G", bitlinear_forward_grouped(5, Ws, Gs, Ns, K, Q, F, S, M, Ys, BITLINEAR_BF16, P, 1 << 20,
                                                nullptr),
         BITLINEAR_ERR_SHAPE);
  const int64_t Nbad[2] = {N, 0};
  expect("grouped N", bitlinear_forward_grouped(2, Ws, Gs, Nbad, K, Q, F, S, M, Ys, BITLINEAR_BF16, P, 1 << 20,
                                                nullptr),
         BITLINEAR_ERR_SHAPE);
  expect("base3 M", bitlinear_forward_base3(W, F, N, K, Q, F, S, BITLINEAR_BASE3_MAX_M + 1, P, BITLINEAR_BF16,
                                            nullptr),
         BITLINEAR_ERR_SHAPE);
  expect_value("status string", std::string(bitlinear_status_string((bitlinear_status)99)) == "unknown status", 1);

  if (no_gpu) {
    expect("forward no device", bitlinear_forward(W, F, N, K, Q, F, S, M, P, BITLINEAR_BF16, P, 1 << 20, nullptr),
           BITLINEAR_ERR_NO_DEVICE);
    expect("pack no device", bitlinear_pack_weights(F, N, K, (uint8_t*)P, (float*)P, P, 1 << 20, nullptr),
           BITLINEAR_ERR_NO_DEVICE);
    expect("noalloc no device", bitlinear_forward_f32_noalloc(W, F, N, K, F, 1, P, BITLINEAR_BF16, nullptr,
                                                              nullptr, nullptr, nullptr),
           BITLINEAR_ERR_NO_DEVICE);
  }
  if (failures) return 1;
  std::printf("abi_check ok (%s)\n", no_gpu ? "no device visible" : "device visible: validation only");
  return 0;
}
