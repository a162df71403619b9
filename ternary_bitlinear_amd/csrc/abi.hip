// C ABI of the BitLinear library: argument validation, device checks and
// dispatch to the kernel launchers.  Every check that can fail runs before
// the first HIP call of an entry point.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/bitlinear.h"
#include "kernels.hpp"

static_assert(BITLINEAR_MAX_GROUP == bl::kMaxGroupProjections, "group size");
static_assert(BITLINEAR_BASE3_MAX_M == bl::kBase3MaxTokens, "base-3 tokens");

namespace {

thread_local std::string g_last_error;

bitlinear_status fail(bitlinear_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
bitlinear_status fail(bitlinear_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// The int a C caller passed for an enum parameter.  Any int is a valid C
// argument, but in C++ reading a value outside the enumerators' range through
// the enum type is undefined, so validation reads the bytes as an int.
template <typename E>
int enum_value(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "enum passed as int");
  int v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}

bool dtype_ok(const bitlinear_dtype& d) {
  const int v = enum_value(d);
  return v == BITLINEAR_F32 || v == BITLINEAR_BF16 || v == BITLINEAR_I32;
}

bool shape_ok_k(int64_t K) { return K >= 16 && K % 16 == 0 && K <= BITLINEAR_MAX_K; }
constexpr int64_t kMaxDim = 0x7fffffff;

// Per-device result of the architecture check: 0 unknown, 1 gfx950, 2 other.
std::atomic<int> g_arch_ok[64];

bitlinear_status check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) {
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count == 0)
      return fail(BITLINEAR_ERR_NO_DEVICE, "no HIP device visible");
    return fail(BITLINEAR_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  }
  if (dev >= 64) return fail(BITLINEAR_ERR_ARCH, "device index %d not supported", dev);
  int st = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return fail(BITLINEAR_ERR_HIP, "hipGetDeviceProperties failed: %s", hipGetErrorString(e));
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_ok[dev].store(st, std::memory_order_relaxed);
  }
  if (st != 1) return fail(BITLINEAR_ERR_ARCH, "device %d is not gfx950", dev);
  return BITLINEAR_OK;
}

bitlinear_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(BITLINEAR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  g_last_error.clear();
  return BITLINEAR_OK;
}

}  // namespace

extern "C" {

int bitlinear_abi_version(void) { return BITLINEAR_ABI_VERSION; }

size_t bitlinear_packed_bytes(int64_t N, int64_t K) {
  if (N < 1 || N > kMaxDim || !shape_ok_k(K)) return 0;
  return (size_t)(N * (K / 4));
}

size_t bitlinear_pack_workspace_bytes(int64_t N, int64_t K) {
  if (N < 1 || N > kMaxDim || !shape_ok_k(K) || N * K > kMaxDim) return 0;
  return bl::pack_workspace_bytes(N, K);
}

size_t bitlinear_forward_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || M > kMaxDim || N < 1 || N > kMaxDim || !shape_ok_k(K)) return 0;
  return bl::forward_workspace_bytes(M, N, K);
}

bitlinear_status bitlinear_pack_weights(const float* W, int64_t N, int64_t K, uint8_t* W_packed,
                                        float* gamma, void* workspace, size_t workspace_bytes,
                                        void* stream) {
  if (!W || !W_packed || !gamma) return fail(BITLINEAR_ERR_NULL, "pack_weights: NULL buffer");
  if (N < 1 || N > kMaxDim || !shape_ok_k(K) || N * K > kMaxDim)
    return fail(BITLINEAR_ERR_SHAPE, "pack_weights: invalid shape N=%lld K=%lld (need N>=1, "
                "K%%16==0, 16<=K<=%d, N*K<2^31)", (long long)N, (long long)K, BITLINEAR_MAX_K);
  if (!aligned(W, 16) || !aligned(W_packed, 16) || !aligned(gamma, 4))
    return fail(BITLINEAR_ERR_ALIGN, "pack_weights: W and W_packed need 16-byte alignment, "
                "gamma 4-byte");
  const size_t need = bl::pack_workspace_bytes(N, K);
  if (!workspace || workspace_bytes < need)
    return fail(BITLINEAR_ERR_WORKSPACE, "pack_weights: workspace of %zu bytes needed, got %zu",
                need, workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 16)) return fail(BITLINEAR_ERR_ALIGN, "pack_weights: workspace alignment");
  bitlinear_status s = check_device();
  if (s != BITLINEAR_OK) return s;
  return launched(bl::launch_pack(W, N, K, W_packed, gamma, workspace,
                                  reinterpret_cast<hipStream_t>(stream)),
                  "pack_weights launch");
}

bitlinear_status bitlinear_quant_acts(const float* X, int64_t M, int64_t K, int8_t* X_q,
                                      float* x_scale, int32_t* x_sum, void* stream) {
  return bitlinear_quant_acts_bits(X, M, K, 8, X_q, x_scale, x_sum, stream);
}

bitlinear_status bitlinear_quant_acts_bits(const float* X, int64_t M, int64_t K, int bits,
                                           int8_t* X_q, float* x_scale, int32_t* x_sum,
                                           void* stream) {
  if (!X || !X_q || !x_scale || !x_sum) return fail(BITLINEAR_ERR_NULL, "quant_acts: NULL buffer");
  if (bits != 8 && bits != 4)
    return fail(BITLINEAR_ERR_DTYPE, "quant_acts: activation bits %d (8 or 4)", bits);
  if (M < 1 || M > kMaxDim || !shape_ok_k(K))
    return fail(BITLINEAR_ERR_SHAPE, "quant_acts: invalid shape M=%lld K=%lld", (long long)M,
                (long long)K);
  if (!aligned(X, 16) || !aligned(X_q, 16) || !aligned(x_scale, 4) || !aligned(x_sum, 4))
    return fail(BITLINEAR_ERR_ALIGN, "quant_acts: X and X_q need 16-byte alignment");
  bitlinear_status s = check_device();
  if (s != BITLINEAR_OK) return s;
  return launched(bl::launch_quant(X, M, K, X_q, x_scale, x_sum,
                                   reinterpret_cast<hipStream_t>(stream), bits),
                  "quant_acts launch");
}

bitlinear_status bitlinear_forward(const uint8_t* W_packed, const float* gamma, int64_t N,
                                   int64_t K, const int8_t* X_q, const float* x_scale,
                                   const int32_t* x_sum, int64_t M, void* Y,
                                   bitlinear_dtype y_dtype, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if (!W_packed || !gamma || !X_q || !x_scale || !x_sum || !Y)
    return fail(BITLINEAR_ERR_NULL, "forward: NULL buffer");
  if (M < 1 || M > kMaxDim || N < 1 || N > kMaxDim || !shape_ok_k(K))
    return fail(BITLINEAR_ERR_SHAPE, "forward: invalid shape M=%lld N=%lld K=%lld", (long long)M,
                (long long)N, (long long)K);
  if (!dtype_ok(y_dtype))
    return fail(BITLINEAR_ERR_DTYPE, "forward: unknown y_dtype %d", enum_value(y_dtype));
  const uintptr_t ya = y_dtype == BITLINEAR_BF16 ? 2 : 4;
  if (!aligned(W_packed, 16) || !aligned(X_q, 16) || !aligned(gamma, 4) || !aligned(x_scale, 4) ||
      !aligned(x_sum, 4) || !aligned(Y, ya))
    return fail(BITLINEAR_ERR_ALIGN, "forward: W_packed/X_q need 16-byte alignment, Y its "
                "element size");
  const size_t need = bl::forward_workspace_bytes(M, N, K);
  if (need && (!workspace || workspace_bytes < need))
    return fail(BITLINEAR_ERR_WORKSPACE, "forward: workspace of %zu bytes needed, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  if (need && !aligned(workspace, 16)) return fail(BITLINEAR_ERR_ALIGN, "forward: workspace alignment");
  bitlinear_status s = check_device();
  if (s != BITLINEAR_OK) return s;
  return launched(bl::launch_forward(W_packed, gamma, N, K, X_q, x_scale, x_sum, M, Y,
                                     (int)y_dtype, need ? workspace : nullptr,
                                     reinterpret_cast<hipStream_t>(stream)),
                  "forward launch");
}

namespace {
// fp32 activations in: the quantiser (after an RMS normalisation with gain
// norm_g when that is not null) and the projection.
// noalloc: the workspace is the library's own scratch array (workspace and
// workspace_bytes unused); the call is refused when it needs more.
bitlinear_status forward_f32_impl(const char* who, const uint8_t* W_packed, const float* gamma,
                                  int64_t N, int64_t K, const float* X, const float* norm_g,
                                  int64_t M, void* Y, bitlinear_dtype y_dtype, int8_t* X_q_out,
                                  float* x_scale_out, int32_t* x_sum_out, void* workspace,
                                  size_t workspace_bytes, void* stream, bool noalloc = false) {
  if (!W_packed || !gamma || !X || !Y) return fail(BITLINEAR_ERR_NULL, "%s: NULL buffer", who);
  const int given = (X_q_out != nullptr) + (x_scale_out != nullptr) + (x_sum_out != nullptr);
  if (given != 0 && given != 3)
    return fail(BITLINEAR_ERR_NULL, "%s: X_q_out, x_scale_out and x_sum_out go together", who);
  if (M < 1 || M > kMaxDim || N < 1 || N > kMaxDim || !shape_ok_k(K))
    return fail(BITLINEAR_ERR_SHAPE, "%s: invalid shape M=%lld N=%lld K=%lld", who,
                (long long)M, (long long)N, (long long)K);
  if (!dtype_ok(y_dtype))
    return fail(BITLINEAR_ERR_DTYPE, "%s: unknown y_dtype %d", who, enum_value(y_dtype));
  const uintptr_t ya = y_dtype == BITLINEAR_BF16 ? 2 : 4;
  if (!aligned(W_packed, 16) || !aligned(X, 16) || !aligned(gamma, 4) || !aligned(Y, ya) ||
      (norm_g && !aligned(norm_g, 16)) ||
      (X_q_out && (!aligned(X_q_out, 16) || !aligned(x_scale_out, 4) || !aligned(x_sum_out, 4))))
    return fail(BITLINEAR_ERR_ALIGN, "%s: W_packed, X, the gain and X_q_out need 16-byte "
                "alignment, Y its element size", who);
  // With the quantiser outputs given, the workspace is needed only for the
  // projection's own part (same layout: it follows the quantiser region).
  const bool norm = norm_g != nullptr;
  const bool proj_ws = M > 16 && bl::forward_workspace_bytes(M, N, K) > 0;
  if (noalloc) {
    // the scratch array takes the workspace's whole layout (quantiser region,
    // then the projection's part) whether or not the outputs are given
    const size_t need = bl::forward_f32_workspace_bytes(M, N, K, norm);
    if (need > bl::noalloc_scratch_bytes())
      return fail(BITLINEAR_ERR_WORKSPACE, "%s: M=%lld N=%lld K=%lld needs %zu bytes of scratch; "
                  "the library's array holds %zu (call bitlinear_forward_f32 with a workspace)",
                  who, (long long)M, (long long)N, (long long)K, need, bl::noalloc_scratch_bytes());
    bitlinear_status s = check_device();
    if (s != BITLINEAR_OK) return s;
    return launched(bl::launch_forward_f32_noalloc(W_packed, gamma, N, K, X, M, Y, (int)y_dtype,
                                                   X_q_out, x_scale_out, x_sum_out,
                                                   reinterpret_cast<hipStream_t>(stream)),
                    "forward launch");
  }
  const size_t need = (given && !proj_ws) ? 0 : bl::forward_f32_workspace_bytes(M, N, K, norm);
  if (need && (!workspace || workspace_bytes < need))
    return fail(BITLINEAR_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, got %zu", who,
                need, workspace ? workspace_bytes : (size_t)0);
  if (need && !aligned(workspace, 16))
    return fail(BITLINEAR_ERR_ALIGN, "%s: workspace alignment", who);
  bitlinear_status s = check_device();
  if (s != BITLINEAR_OK) return s;
  return launched(bl::launch_forward_f32(W_packed, gamma, N, K, X, norm_g, M, Y, (int)y_dtype,
                                         X_q_out, x_scale_out, x_sum_out, workspace,
                                         reinterpret_cast<hipStream_t>(stream)),
                  "forward launch");
}

size_t forward_f32_ws(int64_t M, int64_t N, int64_t K, bool norm) {
  if (M < 1 || M > kMaxDim || N < 1 || N > kMaxDim || !shape_ok_k(K)) return 0;
  return bl::forward_f32_workspace_bytes(M, N, K, norm);
}
}  // namespace

size_t bitlinear_forward_f32_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  return forward_f32_ws(M, N, K, false);
}

bitlinear_status bitlinear_forward_f32(const uint8_t* W_packed, const float* gamma, int64_t N,
                                       int64_t K, const float* X, int64_t M, void* Y,
                                       bitlinear_dtype y_dtype, int8_t* X_q_out,
                                       float* x_scale_out, int32_t* x_sum_out, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  return forward_f32_impl("forward_f32", W_packed, gamma, N, K, X, nullptr, M, Y, y_dtype,
                          X_q_out, x_scale_out, x_sum_out, workspace, workspace_bytes, stream);
}

bitlinear_status bitlinear_forward_f32_noalloc(const uint8_t* W_packed, const float* gamma,
                                               int64_t N, int64_t K, const float* X, int64_t M,
                                               void* Y, bitlinear_dtype y_dtype, int8_t* X_q_out,
                                               float* x_scale_out, int32_t* x_sum_out,
                                               void* stream) {
  return forward_f32_impl("forward_f32_noalloc", W_packed, gamma, N, K, X, nullptr, M, Y, y_dtype,
                          X_q_out, x_scale_out, x_sum_out, nullptr, 0, stream, true);
}

// ---- RMS normalisation before the quantiser -------------------------------------

bitlinear_status bitlinear_rmsnorm_quant(const float* X, const float* norm_g, int64_t M,
                                         int64_t K, int8_t* X_q, float* x_scale, int32_t* x_sum,
                                         void* stream) {
  if (!X || !norm_g || !X_q || !x_scale || !x_sum)
    return fail(BITLINEAR_ERR_NULL, "rmsnorm_quant: NULL buffer");
  if (M < 1 || M > kMaxDim || !shape_ok_k(K))
    return fail(BITLINEAR_ERR_SHAPE, "rmsnorm_quant: invalid shape M=%lld K=%lld", (long long)M,
                (long long)K);
  if (!aligned(X, 16) || !aligned(norm_g, 16) || !aligned(X_q, 16) || !aligned(x_scale, 4) ||
      !aligned(x_sum, 4))
    return fail(BITLINEAR_ERR_ALIGN, "rmsnorm_quant: X, the gain and X_q need 16-byte alignment");
  bitlinear_status s = check_device();
  if (s != BITLINEAR_OK) return s;
  return launched(bl::launch_rmsnorm_quant(X, norm_g, M, K, X_q, x_scale, x_sum,
                                           reinterpret_cast<hipStream_t>(stream)),
                  "rmsnorm_quant launch");
}

size_t bitlinear_forward_rmsnorm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  return forward_f32_ws(M, N, K, true);
}

bitlinear_status bitlinear_forward_rmsnorm(const uint8_t* W_packed, const float* gamma, int64_t N,
                                           int64_t K, const float* X, const float* norm_g,
                                           int64_t M, void* Y, bitlinear_dtype y_dtype,
                                           int8_t* X_q_out, float* x_scale_out,
                                           int32_t* x_sum_out, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  if (!norm_g) return fail(BITLINEAR_ERR_NULL, "forward_rmsnorm: NULL gain");
  return forward_f32_impl("forward_rmsnorm", W_packed, gamma, N, K, X, norm_g, M, Y, y_dtype,
                          X_q_out, x_scale_out, x_sum_out, workspace, workspace_bytes, stream);
}

// ---- several projections of one activation matrix -----------------------------

namespace {
bitlinear_status check_group(const char* who, int G, const uint8_t* const* W_packed,
                             const float* const* gamma, const int64_t* N, int64_t K, int64_t M,
                             void* const* Y, bitlinear_dtype y_dtype) {
  if (G < 1 || G > BITLINEAR_MAX_GROUP)
    return fail(BITLINEAR_ERR_SHAPE, "%s: G=%d outside 1..%d", who, G, BITLINEAR_MAX_GROUP);
  if (!W_packed || !gamma || !N || !Y) return fail(BITLINEAR_ERR_NULL, "%s: NULL array", who);
  if (M < 1 || M > kMaxDim || !shape_ok_k(K))
    return fail(BITLINEAR_ERR_SHAPE, "%s: invalid shape M=%lld K=%lld", who, (long long)M,
                (long long)K);
  if (!dtype_ok(y_dtype))
    return fail(BITLINEAR_ERR_DTYPE, "%s: unknown y_dtype %d", who, enum_value(y_dtype));
  const uintptr_t ya = y_dtype == BITLINEAR_BF16 ? 2 : 4;
  for (int g = 0; g < G; ++g) {
    if (!W_packed[g] || !gamma[g] || !Y[g])
      return fail(BITLINEAR_ERR_NULL, "%s: NULL buffer of projection %d", who, g);
    if (N[g] < 1 || N[g] > kMaxDim)
      return fail(BITLINEAR_ERR_SHAPE, "%s: invalid N=%lld of projection %d", who,
                  (long long)N[g], g);
    if (!aligned(W_packed[g], 16) || !aligned(gamma[g], 4) || !aligned(Y[g], ya))
      return fail(BITLINEAR_ERR_ALIGN, "%s: projection %d: W_packed needs 16-byte alignment, "
                  "Y its element size", who, g);
  }
  return BITLINEAR_OK;
}
}  // namespace

size_t bitlinear_forward_grouped_workspace_bytes(int64_t M, int G, const int64_t* N, int64_t K) {
  if (G < 1 || G > BITLINEAR_MAX_GROUP || !N || M < 1 || M > kMaxDim || !shape_ok_k(K)) return 0;
  for (int g = 0; g < G; ++g)
    if (N[g] < 1 || N[g] > kMaxDim) return 0;
  return bl::forward_grouped_workspace_bytes(M, G, N, K);
}

bitlinear_status bitlinear_forward_grouped(int G, const uint8_t* const* W_packed,
                                           const float* const* gamma, const int64_t* N,
                                           int64_t K, const int8_t* X_q, const float* x_scale,
                                           const int32_t* x_sum, int64_t M, void* const* Y,
                                           bitlinear_dtype y_dtype, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  bitlinear_status s = check_group("forward_grouped", G, W_packed, gamma, N, K, M, Y, y_dtype);
  if (s != BITLINEAR_OK) return s;
  if (!X_q || !x_scale || !x_sum) return fail(BITLINEAR_ERR_NULL, "forward_grouped: NULL buffer");
  if (!aligned(X_q, 16) || !aligned(x_scale, 4) || !aligned(x_sum, 4))
    return fail(BITLINEAR_ERR_ALIGN, "forward_grouped: X_q needs 16-byte alignment");
  const size_t need = bl::forward_grouped_workspace_bytes(M, G, N, K);
  if (need && (!workspace || workspace_bytes < need))
    return fail(BITLINEAR_ERR_WORKSPACE, "forward_grouped: workspace of %zu bytes needed, got %zu",
                need, workspace ? workspace_bytes : (size_t)0);
  if (need && !aligned(workspace, 16))
    return fail(BITLINEAR_ERR_ALIGN, "forward_grouped: workspace alignment");
  s = check_device();
  if (s != BITLINEAR_OK) return s;
  return launched(bl::launch_forward_grouped(G, W_packed, gamma, N, K, X_q, x_scale, x_sum, M, Y,
                                             (int)y_dtype, need ? workspace : nullptr,
                                             reinterpret_cast<hipStream_t>(stream)),
                  "forward_grouped launch");
}

namespace {
size_t forward_f32_grouped_ws(int64_t M, int G, const int64_t* N, int64_t K, bool norm) {
  if (G < 1 || G > BITLINEAR_MAX_GROUP || !N || M < 1 || M > kMaxDim || !shape_ok_k(K)) return 0;
  for (int g = 0; g < G; ++g)
    if (N[g] < 1 || N[g] > kMaxDim) return 0;
  return bl::forward_f32_grouped_workspace_bytes(M, G, N, K, norm);
}

bitlinear_status forward_f32_grouped_impl(const char* who, int G, const uint8_t* const* W_packed,
                                          const float* const* gamma, const int64_t* N, int64_t K,
                                          const float* X, const float* norm_g, int64_t M,
                                          void* const* Y, bitlinear_dtype y_dtype,
                                          int8_t* X_q_out, float* x_scale_out,
                                          int32_t* x_sum_out, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  bitlinear_status s = check_group(who, G, W_packed, gamma, N, K, M, Y, y_dtype);
  if (s != BITLINEAR_OK) return s;
  if (!X) return fail(BITLINEAR_ERR_NULL, "%s: NULL X", who);
  const int given = (X_q_out != nullptr) + (x_scale_out != nullptr) + (x_sum_out != nullptr);
  if (given != 0 && given != 3)
    return fail(BITLINEAR_ERR_NULL, "%s: X_q_out, x_scale_out and x_sum_out go together", who);
  if (!aligned(X, 16) || (norm_g && !aligned(norm_g, 16)) ||
      (X_q_out && (!aligned(X_q_out, 16) || !aligned(x_scale_out, 4) || !aligned(x_sum_out, 4))))
    return fail(BITLINEAR_ERR_ALIGN, "%s: X, the gain and X_q_out need 16-byte alignment", who);
  // With the quantiser outputs given, the workspace is needed only for the
  // projections' own part (same layout: it follows the quantiser region).
  const bool norm = norm_g != nullptr;
  const bool proj_ws = M > 16 && bl::forward_grouped_workspace_bytes(M, G, N, K) > 0;
  const size_t need =
      (given && !proj_ws) ? 0 : bl::forward_f32_grouped_workspace_bytes(M, G, N, K, norm);
  if (need && (!workspace || workspace_bytes < need))
    return fail(BITLINEAR_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, got %zu", who,
                need, workspace ? workspace_bytes : (size_t)0);
  if (need && !aligned(workspace, 16))
    return fail(BITLINEAR_ERR_ALIGN, "%s: workspace alignment", who);
  s = check_device();
  if (s != BITLINEAR_OK) return s;
  return launched(bl::launch_forward_f32_grouped(G, W_packed, gamma, N, K, X, norm_g, M, Y,
                                                 (int)y_dtype, X_q_out, x_scale_out, x_sum_out,
                                                 workspace, reinterpret_cast<hipStream_t>(stream)),
                  "grouped forward launch");
}
}  // namespace

size_t bitlinear_forward_f32_grouped_workspace_bytes(int64_t M, int G, const int64_t* N,
                                                     int64_t K) {
  return forward_f32_grouped_ws(M, G, N, K, false);
}

bitlinear_status bitlinear_forward_f32_grouped(int G, const uint8_t* const* W_packed,
                                               const float* const* gamma, const int64_t* N,
                                               int64_t K, const float* X, int64_t M,
                                               void* const* Y, bitlinear_dtype y_dtype,
                                               int8_t* X_q_out, float* x_scale_out,
                                               int32_t* x_sum_out, void* workspace,
                                               size_t workspace_bytes, void* stream) {
  return forward_f32_grouped_impl("forward_f32_grouped", G, W_packed, gamma, N, K, X, nullptr, M,
                                  Y, y_dtype, X_q_out, x_scale_out, x_sum_out, workspace,
                                  workspace_bytes, stream);
}

size_t bitlinear_forward_rmsnorm_grouped_workspace_bytes(int64_t M, int G, const int64_t* N,
                                                         int64_t K) {
  return forward_f32_grouped_ws(M, G, N, K, true);
}

bitlinear_status bitlinear_forward_rmsnorm_grouped(int G, const uint8_t* const* W_packed,
                                                   const float* const* gamma, const int64_t* N,
                                                   int64_t K, const float* X,
                                                   const float* norm_g, int64_t M,
                                                   void* const* Y, bitlinear_dtype y_dtype,
                                                   int8_t* X_q_out, float* x_scale_out,
                                                   int32_t* x_sum_out, void* workspace,
                                                   size_t workspace_bytes, void* stream) {
  if (!norm_g) return fail(BITLINEAR_ERR_NULL, "forward_rmsnorm_grouped: NULL gain");
  return forward_f32_grouped_impl("forward_rmsnorm_grouped", G, W_packed, gamma, N, K, X, norm_g,
                                  M, Y, y_dtype, X_q_out, x_scale_out, x_sum_out, workspace,
                                  workspace_bytes, stream);
}

// ---- several projections with their own activations ----------------------------

namespace {
bool multi_shapes_ok(int64_t M, int G, const int64_t* N, const int64_t* K) {
  if (G < 1 || G > BITLINEAR_MAX_GROUP || !N || !K || M < 1 || M > kMaxDim) return false;
  for (int g = 0; g < G; ++g)
    if (N[g] < 1 || N[g] > kMaxDim || !shape_ok_k(K[g])) return false;
  return true;
}
}  // namespace

int bitlinear_forward_f32_multi_kernel(int64_t M, int G, const int64_t* N, const int64_t* K) {
  if (!multi_shapes_ok(M, G, N, K)) return -BITLINEAR_ERR_SHAPE;
  static_assert(BITLINEAR_KERNEL_STREAM == bl::kKernelStream, "kernel ids");
  return bl::stream_multi_ok(M, G, N, K) ? (BITLINEAR_KERNEL_STREAM | BITLINEAR_KERNEL_FUSED_QUANT)
                                         : 0;
}

size_t bitlinear_forward_f32_multi_workspace_bytes(int64_t M, int G, const int64_t* N,
                                                   const int64_t* K) {
  if (!multi_shapes_ok(M, G, N, K)) return 0;
  return bl::forward_f32_multi_workspace_bytes(M, G, N, K);
}

bitlinear_status bitlinear_forward_f32_multi(int G, const uint8_t* const* W_packed,
                                             const float* const* gamma, const int64_t* N,
                                             const int64_t* K, const float* const* X, int64_t M,
                                             void* const* Y, bitlinear_dtype y_dtype,
                                             void* workspace, size_t workspace_bytes,
                                             void* stream) {
  if (G < 1 || G > BITLINEAR_MAX_GROUP)
    return fail(BITLINEAR_ERR_SHAPE, "forward_f32_multi: G=%d outside 1..%d", G,
                BITLINEAR_MAX_GROUP);
  if (!W_packed || !gamma || !N || !K || !X || !Y)
    return fail(BITLINEAR_ERR_NULL, "forward_f32_multi: NULL array");
  if (!multi_shapes_ok(M, G, N, K))
    return fail(BITLINEAR_ERR_SHAPE, "forward_f32_multi: invalid shape (M=%lld; every N >= 1, "
                "K %% 16 == 0, 16 <= K <= %d)", (long long)M, BITLINEAR_MAX_K);
  if (!dtype_ok(y_dtype))
    return fail(BITLINEAR_ERR_DTYPE, "forward_f32_multi: unknown y_dtype %d", enum_value(y_dtype));
  const uintptr_t ya = y_dtype == BITLINEAR_BF16 ? 2 : 4;
  for (int g = 0; g < G; ++g) {
    if (!W_packed[g] || !gamma[g] || !X[g] || !Y[g])
      return fail(BITLINEAR_ERR_NULL, "forward_f32_multi: NULL buffer of projection %d", g);
    if (!aligned(W_packed[g], 16) || !aligned(X[g], 16) || !aligned(gamma[g], 4) ||
        !aligned(Y[g], ya))
      return fail(BITLINEAR_ERR_ALIGN, "forward_f32_multi: projection %d: W_packed and X need "
                  "16-byte alignment, Y its element size", g);
  }
  const size_t need = bl::forward_f32_multi_workspace_bytes(M, G, N, K);
  if (need && (!workspace || workspace_bytes < need))
    return fail(BITLINEAR_ERR_WORKSPACE, "forward_f32_multi: workspace of %zu bytes needed, got %zu",
                need, workspace ? workspace_bytes : (size_t)0);
  if (need && !aligned(workspace, 16))
    return fail(BITLINEAR_ERR_ALIGN, "forward_f32_multi: workspace alignment");
  bitlinear_status s = check_device();
  if (s != BITLINEAR_OK) return s;
  return launched(bl::launch_forward_f32_multi(G, W_packed, gamma, N, K, X, M, Y, (int)y_dtype,
                                               need ? workspace : nullptr,
                                               reinterpret_cast<hipStream_t>(stream)),
                  "forward_f32_multi launch");
}

size_t bitlinear_packed3_bytes(int64_t N, int64_t K) {
  if (N < 1 || N > kMaxDim || !shape_ok_k(K)) return 0;
  return (size_t)N * bl::packed3_row_bytes(K);
}

bitlinear_status bitlinear_pack_weights_base3(const float* W, int64_t N, int64_t K,
                                              uint8_t* W_packed3, float* gamma, void* workspace,
                                              size_t workspace_bytes, void* stream) {
  if (!W || !W_packed3 || !gamma) return fail(BITLINEAR_ERR_NULL, "pack_weights_base3: NULL buffer");
  if (N < 1 || N > kMaxDim || !shape_ok_k(K) || N * K > kMaxDim)
    return fail(BITLINEAR_ERR_SHAPE, "pack_weights_base3: invalid shape N=%lld K=%lld (need N>=1, "
                "K%%16==0, 16<=K<=%d, N*K<2^31)", (long long)N, (long long)K, BITLINEAR_MAX_K);
  if (!aligned(W, 16) || !aligned(W_packed3, 16) || !aligned(gamma, 4))
    return fail(BITLINEAR_ERR_ALIGN, "pack_weights_base3: W and W_packed3 need 16-byte alignment, "
                "gamma 4-byte");
  const size_t need = bl::pack_workspace_bytes(N, K);
  if (!workspace || workspace_bytes < need)
    return fail(BITLINEAR_ERR_WORKSPACE, "pack_weights_base3: workspace of %zu bytes needed, got %zu",
                need, workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 16))
    return fail(BITLINEAR_ERR_ALIGN, "pack_weights_base3: workspace alignment");
  bitlinear_status s = check_device();
  if (s != BITLINEAR_OK) return s;
  return launched(bl::launch_pack3(W, N, K, W_packed3, gamma, workspace,
                                   reinterpret_cast<hipStream_t>(stream)),
                  "pack_weights_base3 launch");
}

bitlinear_status bitlinear_forward_base3(const uint8_t* W_packed3, const float* gamma, int64_t N,
                                         int64_t K, const int8_t* X_q, const float* x_scale,
                                         const int32_t* x_sum, int64_t M, void* Y,
                                         bitlinear_dtype y_dtype, void* stream) {
  if (!W_packed3 || !gamma || !X_q || !x_scale || !x_sum || !Y)
    return fail(BITLINEAR_ERR_NULL, "forward_base3: NULL buffer");
  if (M < 1 || M > BITLINEAR_BASE3_MAX_M || N < 1 || N > kMaxDim || !shape_ok_k(K))
    return fail(BITLINEAR_ERR_SHAPE, "forward_base3: invalid shape M=%lld N=%lld K=%lld (need "
                "1<=M<=%d)", (long long)M, (long long)N, (long long)K, BITLINEAR_BASE3_MAX_M);
  if (!dtype_ok(y_dtype))
    return fail(BITLINEAR_ERR_DTYPE, "forward_base3: unknown y_dtype %d", enum_value(y_dtype));
  const uintptr_t ya = y_dtype == BITLINEAR_BF16 ? 2 : 4;
  if (!aligned(W_packed3, 16) || !aligned(X_q, 16) || !aligned(gamma, 4) ||
      !aligned(x_scale, 4) || !aligned(x_sum, 4) || !aligned(Y, ya))
    return fail(BITLINEAR_ERR_ALIGN, "forward_base3: W_packed3/X_q need 16-byte alignment, Y its "
                "element size");
  bitlinear_status s = check_device();
  if (s != BITLINEAR_OK) return s;
  return launched(bl::launch_forward_b3(W_packed3, gamma, N, K, X_q, x_scale, x_sum, M, Y,
                                        (int)y_dtype, reinterpret_cast<hipStream_t>(stream)),
                  "forward_base3 launch");
}

bitlinear_status bitlinear_base3_to_blt2(const uint8_t* W_packed3, int64_t N, int64_t K,
                                         uint8_t* W_packed, void* stream) {
  if (!W_packed3 || !W_packed) return fail(BITLINEAR_ERR_NULL, "base3_to_blt2: NULL buffer");
  if (N < 1 || N > kMaxDim || !shape_ok_k(K))
    return fail(BITLINEAR_ERR_SHAPE, "base3_to_blt2: invalid shape N=%lld K=%lld", (long long)N,
                (long long)K);
  if (!aligned(W_packed3, 16) || !aligned(W_packed, 16))
    return fail(BITLINEAR_ERR_ALIGN, "base3_to_blt2: both buffers need 16-byte alignment");
  bitlinear_status s = check_device();
  if (s != BITLINEAR_OK) return s;
  return launched(bl::launch_b3_to_b2(W_packed3, N, K, W_packed,
                                      reinterpret_cast<hipStream_t>(stream)),
                  "base3_to_blt2 launch");
}

int bitlinear_forward_kernel(int entry, int64_t M, int G, const int64_t* N, int64_t K) {
  if (entry < 0 || entry > 2 || G < 1 || G > BITLINEAR_MAX_GROUP || !N || M < 1 ||
      M > kMaxDim || !shape_ok_k(K))
    return -BITLINEAR_ERR_SHAPE;
  for (int g = 0; g < G; ++g)
    if (N[g] < 1 || N[g] > kMaxDim) return -BITLINEAR_ERR_SHAPE;
  static_assert(BITLINEAR_KERNEL_DECODE_DOT == bl::kKernelDecodeDot &&
                    BITLINEAR_KERNEL_DECODE == bl::kKernelDecode &&
                    BITLINEAR_KERNEL_SKINNY == bl::kKernelSkinny &&
                    BITLINEAR_KERNEL_GEMM == bl::kKernelGemm,
                "kernel ids");
  return bl::forward_kernel(entry, M, G, N, K);
}

const char* bitlinear_status_string(bitlinear_status s) {
  switch (enum_value(s)) {
    case BITLINEAR_OK: return "ok";
    case BITLINEAR_ERR_NULL: return "null pointer";
    case BITLINEAR_ERR_SHAPE: return "invalid shape";
    case BITLINEAR_ERR_ALIGN: return "misaligned pointer";
    case BITLINEAR_ERR_DTYPE: return "invalid dtype";
    case BITLINEAR_ERR_NO_DEVICE: return "no HIP device";
    case BITLINEAR_ERR_ARCH: return "device is not gfx950";
    case BITLINEAR_ERR_WORKSPACE: return "workspace missing or too small";
    case BITLINEAR_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* bitlinear_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
