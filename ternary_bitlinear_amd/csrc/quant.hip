// Per-token absmax int8 quantisation of activations.
//
// Page "BitNet b1.58: Mathematical Foundations ..." (llms.blog), section 2,
// "Activation Quantization: Absmax Scaling", per-token variant with the
// symmetric range [-127, 127]:
//   beta = max_k |x_k|,  x~_k = RoundClip(x_k * (127 / (beta + eps)), -127, 127).
// One workgroup per token.  The max is taken on the bit patterns of |x|
// (exact and order-free); the factor is one fp32 add and one correctly rounded
// fp32 divide; each element gets one fp32 multiply; floor(q + 1/2) is taken
// exactly as floor(q) + (q - floor(q) >= 1/2), where q - floor(q) is exact
// for |q| < 2^23.  The file is built without floating-point contraction, so
// the multiply is never fused with the subtraction.
#include "common.hpp"
#include "kernels.hpp"

namespace bl {

namespace {

constexpr int kQuantThreads = 256;

__device__ __forceinline__ int32_t quant1(float x, float inv) {
  const float q = x * inv;
  const float r = floorf(q);
  int32_t v = (int32_t)r + ((q - r) >= 0.5f ? 1 : 0);
  v = max(-127, min(127, v));
  return v;
}

__global__ __launch_bounds__(kQuantThreads) void k_quant_acts(const float* __restrict__ X,
                                                              int64_t K, int8_t* __restrict__ Xq,
                                                              float* __restrict__ x_scale,
                                                              int32_t* __restrict__ x_sum) {
  __shared__ uint32_t s_max[kQuantThreads / kWave];
  __shared__ int32_t s_sum[kQuantThreads / kWave];
  const int64_t m = blockIdx.x;
  const float4* row = reinterpret_cast<const float4*>(X + m * K);
  uint32_t* qrow = reinterpret_cast<uint32_t*>(Xq + m * K);
  const int64_t K4 = K / 4;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;

  uint32_t amax = 0;
  for (int64_t i = threadIdx.x; i < K4; i += kQuantThreads) {
    const float4 f = row[i];
    amax = max(amax, max(max(abs_bits(f.x), abs_bits(f.y)), max(abs_bits(f.z), abs_bits(f.w))));
  }
  amax = wave_max_u32(amax);
  if (lane == 0) s_max[wave] = amax;
  __syncthreads();
  amax = s_max[0];
#pragma unroll
  for (int w = 1; w < kQuantThreads / kWave; ++w) amax = max(amax, s_max[w]);
  const float beta = __uint_as_float(amax);
  const float inv = 127.0f / (beta + 1e-5f);

  int32_t sum = 0;
  for (int64_t i = threadIdx.x; i < K4; i += kQuantThreads) {
    const float4 f = row[i];
    const int32_t a = quant1(f.x, inv), b = quant1(f.y, inv), c = quant1(f.z, inv),
                  d = quant1(f.w, inv);
    sum += a + b + c + d;
    qrow[i] = (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
              ((uint32_t)(d & 0xff) << 24);
  }
  sum = wave_sum_i32(sum);
  if (lane == 0) s_sum[wave] = sum;
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t t = 0;
#pragma unroll
    for (int w = 0; w < kQuantThreads / kWave; ++w) t += s_sum[w];
    x_sum[m] = t;
    x_scale[m] = beta / 127.0f;
  }
}

}  // namespace

hipError_t launch_quant(const float* X, int64_t M, int64_t K, int8_t* X_q, float* x_scale,
                        int32_t* x_sum, hipStream_t stream) {
  k_quant_acts<<<dim3((unsigned)M), dim3(kQuantThreads), 0, stream>>>(X, K, X_q, x_scale, x_sum);
  return hipGetLastError();
}

}  // namespace bl
