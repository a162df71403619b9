// Host-side launchers of the BitLinear kernels (called by the C ABI layer).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

constexpr int64_t kPackWsHeader = 256;   // bytes before the partial sums

size_t pack_workspace_bytes(int64_t N, int64_t K);

hipError_t launch_pack(const float* W, int64_t N, int64_t K, uint8_t* W_packed, float* gamma,
                       void* workspace, hipStream_t stream);

hipError_t launch_quant(const float* X, int64_t M, int64_t K, int8_t* X_q, float* x_scale,
                        int32_t* x_sum, hipStream_t stream,
                        int bits = 8);

// The int8 quantiser over up to kQuantMaxMulti activation matrices [M][K[g]]
// in one launch (the same per-row arithmetic as launch_quant).
constexpr int kQuantMaxMulti = 4;
hipError_t launch_quant_multi(int G, const float* const* X, int64_t M, const int64_t* K,
                              int8_t* const* X_q, float* const* x_scale, int32_t* const* x_sum,
                              hipStream_t stream);

// RMS normalisation with gain G [K], then the same quantiser.
hipError_t launch_rmsnorm_quant(const float* X, const float* G, int64_t M, int64_t K,
                                int8_t* X_q, float* x_scale, int32_t* x_sum, hipStream_t stream);

// Workspace of the projection: split-K partial accumulators for shapes with
// few output tiles and long K, else 0.
size_t forward_workspace_bytes(int64_t M, int64_t N, int64_t K);

// y_dtype: 0 fp32, 1 bf16, 2 int32 (raw accumulators).  `workspace` holds at
// least forward_workspace_bytes(M, N, K) bytes (16-byte aligned) when that is
// non-zero.
hipError_t launch_forward(const uint8_t* W_packed, const float* gamma, int64_t N, int64_t K,
                          const int8_t* X_q, const float* x_scale, const int32_t* x_sum,
                          int64_t M, void* Y, int y_dtype, void* workspace, hipStream_t stream);

// Several projections of one activation matrix (G <= 4; W_packed, gamma, N
// and Y are host arrays of G entries): decode shapes run as one launch over
// all of them, GEMM shapes one projection after another.
size_t forward_grouped_workspace_bytes(int64_t M, int G, const int64_t* N, int64_t K);
hipError_t launch_forward_grouped(int G, const uint8_t* const* W_packed,
                                  const float* const* gamma, const int64_t* N, int64_t K,
                                  const int8_t* X_q, const float* x_scale, const int32_t* x_sum,
                                  int64_t M, void* const* Y, int y_dtype, void* workspace,
                                  hipStream_t stream);
size_t forward_f32_grouped_workspace_bytes(int64_t M, int G, const int64_t* N, int64_t K,
                                           bool norm);
hipError_t launch_forward_f32_grouped(int G, const uint8_t* const* W_packed,
                                      const float* const* gamma, const int64_t* N, int64_t K,
                                      const float* X, const float* norm_g, int64_t M,
                                      void* const* Y, int y_dtype, int8_t* X_q_out,
                                      float* x_scale_out, int32_t* x_sum_out, void* workspace,
                                      hipStream_t stream);
constexpr int kMaxGroupProjections = 4;

// Quantisation fused with the projection (fp32 activations in; norm_g, when
// not null, the gain of an RMS normalisation applied first).  Optional
// X_q_out / x_scale_out / x_sum_out receive the quantiser's outputs (all or
// none).  Unfused shapes use `workspace`: the quantiser region (used only
// when no outputs are given), then the projection's workspace.
size_t forward_f32_workspace_bytes(int64_t M, int64_t N, int64_t K, bool norm);
hipError_t launch_forward_f32(const uint8_t* W_packed, const float* gamma, int64_t N, int64_t K,
                              const float* X, const float* norm_g, int64_t M, void* Y,
                              int y_dtype, int8_t* X_q_out, float* x_scale_out,
                              int32_t* x_sum_out, void* workspace, hipStream_t stream);

// launch_forward_f32 (no normalisation) with the workspace taken from the
// library's own device array (noalloc.hip): no allocation, no caller
// workspace.  The caller checks forward_f32_workspace_bytes(M, N, K, false)
// <= noalloc_scratch_bytes().
size_t noalloc_scratch_bytes();
hipError_t launch_forward_f32_noalloc(const uint8_t* W_packed, const float* gamma, int64_t N,
                                      int64_t K, const float* X, int64_t M, void* Y, int y_dtype,
                                      int8_t* X_q_out, float* x_scale_out, int32_t* x_sum_out,
                                      hipStream_t stream);

// Several projections with their own activations and K (G <= 4; all arrays
// on the host): one persistent launch for a single token (stream_multi_ok),
// else one launch_forward_f32 per projection (the workspace reused in stream
// order).
bool stream_multi_ok(int64_t M, int G, const int64_t* N, const int64_t* K);
size_t forward_f32_multi_workspace_bytes(int64_t M, int G, const int64_t* N, const int64_t* K);
hipError_t launch_forward_f32_multi(int G, const uint8_t* const* W_packed,
                                   const float* const* gamma, const int64_t* N, const int64_t* K,
                                   const float* const* X, int64_t M, void* const* Y, int y_dtype,
                                   void* workspace, hipStream_t stream);

// Base-3 weights (BLT3-v1, five per byte; rows padded to 80 weights).
// launch_pack3 computes gamma and the codes as launch_pack does (same
// workspace); launch_forward_b3 takes 1 <= M <= kBase3MaxTokens tokens;
// launch_b3_to_b2 rewrites BLT3-v1 rows as BLT2-v1 rows (for larger M).
constexpr int kBase3MaxTokens = 16;
size_t packed3_row_bytes(int64_t K);
hipError_t launch_pack3(const float* W, int64_t N, int64_t K, uint8_t* W_packed3, float* gamma,
                        void* workspace, hipStream_t stream);
hipError_t launch_forward_b3(const uint8_t* W_packed3, const float* gamma, int64_t N, int64_t K,
                             const int8_t* X_q, const float* x_scale, const int32_t* x_sum,
                             int64_t M, void* Y, int y_dtype, hipStream_t stream);
hipError_t launch_b3_to_b2(const uint8_t* W_packed3, int64_t N, int64_t K, uint8_t* W_packed,
                           hipStream_t stream);

// The kernel a forward call launches for these sizes (host only): entry 0
// for the pre-quantised projection, 1 for the fp32 one, 2 with the RMS
// normalisation; kKernel* or'ed with 16 when the quantiser runs inside it.
constexpr int kKernelDecodeDot = 1, kKernelDecode = 2, kKernelSkinny = 3, kKernelGemm = 4,
              kKernelStream = 5;
int forward_kernel(int entry, int64_t M, int G, const int64_t* N, int64_t K);

}  // namespace bl
