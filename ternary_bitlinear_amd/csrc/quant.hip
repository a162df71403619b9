// Per-token absmax int8 quantisation of activations, optionally after RMS
// normalisation.
//
// Page "BitNet b1.58: Mathematical Foundations ..." (llms.blog), section 2,
// "Activation Quantization: Absmax Scaling", per-token variant with the
// symmetric range [-127, 127]:
//   beta = max_k |x_k|,  x~_k = RoundClip(x_k * (127 / (beta + eps)), -127, 127).
// One workgroup per token, the row held in registers (one batch of loads).
// The max is taken on the bit patterns of |x| (exact and order-free); the factor is one fp32 add and one correctly rounded
// fp32 divide; each element gets one fp32 multiply; floor(q + 1/2) is taken
// exactly as floor(q) + (q - floor(q) >= 1/2), where q - floor(q) is exact
// for |q| < 2^23.  The file is built without floating-point contraction, so
// the multiply is never fused with the subtraction.
#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace bl {

namespace {

constexpr int kQuantThreads = 256;

// Longer rows take workgroups of 4 x kQuantThreads threads: one workgroup
// (one CU) serves a token, and 16 waves keep 4 times the loads and
// conversions in flight.  Timed on MI355X, one token: the quantiser at
// K = 8192 in 2.25 vs 2.91 us, 12288 in 2.8 vs 3.85 us, 28672 in 4.3 vs
// 6.7 us, 65536 in 7.5 vs 22.3 us; the normalising quantiser at 28672 in
// 6.7 vs 15.4 us, 65536 in 13.4 vs 32.4 us.  The normalising quantiser
// keeps 256 threads up to 12288 values.
constexpr int64_t kQuantWideKPlain = 4096;
constexpr int64_t kQuantWideK = 12288;
constexpr int kQuantWideThreads = 4 * kQuantThreads;

// Block-wide max / sum over T threads (all threads receive the result).
template <int T>
__device__ __forceinline__ uint32_t block_max(uint32_t v, uint32_t* sh) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  v = wave_max_u32(v);
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  v = sh[0];
#pragma unroll
  for (int w = 1; w < T / kWave; ++w) v = max(v, sh[w]);
  return v;
}

template <int T>
__device__ __forceinline__ int32_t block_sum(int32_t v, int32_t* sh) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  v = wave_sum_i32(v);
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  int32_t t = 0;
#pragma unroll
  for (int w = 0; w < T / kWave; ++w) t += sh[w];
  return t;
}

// R float4 per thread held in registers: the row is read once, with every
// load in flight together.  R = 0 selects the looped variant (two passes) for
// rows longer than the register-resident maximum.
// qmax = Q_b - 1: 127 for int8 activations, 7 for 4-bit ones (stored one
// per byte).  The per-element clip to +-127 is inactive at either width:
// |x| (qmax / (beta + eps)) stays below qmax + 1/2.
template <int R, int T>
__device__ __forceinline__ void quant_row(const float* __restrict__ X, int64_t K,
                                          int8_t* __restrict__ Xq, float* __restrict__ x_scale,
                                          int32_t* __restrict__ x_sum, float qmax,
                                          uint32_t* s_max, int32_t* s_sum) {
  const float4* row = reinterpret_cast<const float4*>(X);
  uint32_t* qrow = reinterpret_cast<uint32_t*>(Xq);
  const int64_t K4 = K / 4;

  uint32_t amax = 0;
  int32_t sum = 0;
  if constexpr (R > 0) {
    float4 v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t i = threadIdx.x + (int64_t)r * T;
      v[r] = i < K4 ? row[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
      amax = max(amax, max(max(abs_bits(v[r].x), abs_bits(v[r].y)),
                           max(abs_bits(v[r].z), abs_bits(v[r].w))));
    amax = block_max<T>(amax, s_max);
    const float beta = __uint_as_float(amax);
    const float inv = qmax / (beta + 1e-5f);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t i = threadIdx.x + (int64_t)r * T;
      if (i < K4) qrow[i] = quant4(v[r], inv, sum);
    }
  } else {
    for (int64_t i = threadIdx.x; i < K4; i += T) {
      const float4 f = row[i];
      amax = max(amax, max(max(abs_bits(f.x), abs_bits(f.y)), max(abs_bits(f.z), abs_bits(f.w))));
    }
    amax = block_max<T>(amax, s_max);
    const float beta = __uint_as_float(amax);
    const float inv = qmax / (beta + 1e-5f);
    for (int64_t i = threadIdx.x; i < K4; i += T) qrow[i] = quant4(row[i], inv, sum);
  }
  sum = block_sum<T>(sum, s_sum);
  if (threadIdx.x == 0) {
    *x_sum = sum;
    *x_scale = __uint_as_float(amax) / qmax;
  }
}

template <int R, int T = kQuantThreads>
__global__ __launch_bounds__(T) void k_quant_acts(const float* __restrict__ X,
                                                  int64_t K, int8_t* __restrict__ Xq,
                                                  float* __restrict__ x_scale,
                                                  int32_t* __restrict__ x_sum, float qmax) {
  __shared__ uint32_t s_max[T / kWave];
  __shared__ int32_t s_sum[T / kWave];
  const int64_t m = blockIdx.x;
  quant_row<R, T>(X + m * K, K, Xq + m * K, x_scale + m, x_sum + m, qmax, s_max, s_sum);
}

// Several activation matrices (each with its own K) in one launch: workgroup
// b quantises row b % M of matrix b / M, with the same per-row arithmetic.
// R and T are chosen for the longest row (shorter rows leave registers idle).
struct QuantMulti {
  const float* X[kQuantMaxMulti];
  int64_t K[kQuantMaxMulti];
  int8_t* Xq[kQuantMaxMulti];
  float* xs[kQuantMaxMulti];
  int32_t* xsum[kQuantMaxMulti];
};

template <int R, int T>
__global__ __launch_bounds__(T) void k_quant_acts_multi(QuantMulti q, int64_t M, float qmax) {
  __shared__ uint32_t s_max[T / kWave];
  __shared__ int32_t s_sum[T / kWave];
  const int g = (int)(blockIdx.x / M);
  const int64_t m = blockIdx.x - g * M;
  const float* X = q.X[0];
  int64_t K = q.K[0];
  int8_t* Xq = q.Xq[0];
  float* xs = q.xs[0];
  int32_t* xsum = q.xsum[0];
#pragma unroll
  for (int i = 1; i < kQuantMaxMulti; ++i)
    if (g == i) {
      X = q.X[i]; K = q.K[i]; Xq = q.Xq[i]; xs = q.xs[i]; xsum = q.xsum[i];
    }
  quant_row<R, T>(X + m * K, K, Xq + m * K, xs + m, xsum + m, qmax, s_max, s_sum);
}

// RMS normalisation, then the absmax quantiser, per token (page section 2:
// the activations are RMS-normalised, then quantised to int8).  One
// workgroup per token; thread t holds groups of four t, t + T, ... of the row
// and of the gain (R of them in registers; R = 0: passes over the row for
// rows beyond the register-resident maximum).  The mean of squares is exact,
// rounded once to fp32 (block_mean_square_fast, else _exact), then
// r = 1 / sqrt(ms + eps); the
// normalised values fl32(fl32(x r) g) go through the same absmax, factor and
// per-element rounding as k_quant_acts.
template <int R, int T = kQuantThreads>
__global__ __launch_bounds__(T) void k_rmsnorm_quant(
    const float* __restrict__ X, const float* __restrict__ G, int64_t K, int8_t* __restrict__ Xq,
    float* __restrict__ x_scale, int32_t* __restrict__ x_sum) {
  __shared__ SqShared<T> s_sq;
  __shared__ uint32_t s_max[T / kWave];
  __shared__ int32_t s_sum[T / kWave];
  const int64_t m = blockIdx.x;
  const float4* row = reinterpret_cast<const float4*>(X + m * K);
  const float4* grow = reinterpret_cast<const float4*>(G);
  uint32_t* qrow = reinterpret_cast<uint32_t*>(Xq + m * K);
  const int64_t K4 = K / 4;

  uint32_t amax = 0;
  int32_t sum = 0;
  float inv;
  if constexpr (R > 0) {
    float4 v[R], gv[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t i = threadIdx.x + (int64_t)r * T;
      v[r] = i < K4 ? row[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      gv[r] = i < K4 ? grow[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    auto visit = [&](auto&& f) {
#pragma unroll
      for (int r = 0; r < R; ++r) f(v[r]);
    };
    float ms;
    if (!block_mean_square_fast<T>(visit, (uint32_t)K, s_sq, ms)) {
      ms = block_mean_square_exact<T>(row, K4, (uint32_t)K, s_sq);
#pragma unroll
      for (int r = 0; r < R; ++r) {   // reloaded: nothing held across the exact path
        const int64_t i = threadIdx.x + (int64_t)r * T;
        v[r] = i < K4 ? row[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        gv[r] = i < K4 ? grow[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    const float rr = rms_reciprocal(ms);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      v[r] = rms_apply(v[r], rr, gv[r]);
      amax = max(amax, absmax4(v[r]));
    }
    amax = block_max<T>(amax, s_max);
    inv = 127.0f / (__uint_as_float(amax) + 1e-5f);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t i = threadIdx.x + (int64_t)r * T;
      if (i < K4) qrow[i] = quant4(v[r], inv, sum);
    }
  } else {
    auto visit = [&](auto&& f) {
      for (int64_t i = threadIdx.x; i < K4; i += T) f(row[i]);
    };
    float ms;
    if (!block_mean_square_fast<T>(visit, (uint32_t)K, s_sq, ms))
      ms = block_mean_square_exact<T>(row, K4, (uint32_t)K, s_sq);
    const float rr = rms_reciprocal(ms);
    for (int64_t i = threadIdx.x; i < K4; i += T)
      amax = max(amax, absmax4(rms_apply(row[i], rr, grow[i])));
    amax = block_max<T>(amax, s_max);
    inv = 127.0f / (__uint_as_float(amax) + 1e-5f);
    for (int64_t i = threadIdx.x; i < K4; i += T)
      qrow[i] = quant4(rms_apply(row[i], rr, grow[i]), inv, sum);
  }
  sum = block_sum<T>(sum, s_sum);
  if (threadIdx.x == 0) {
    x_sum[m] = sum;
    x_scale[m] = __uint_as_float(amax) / 127.0f;
  }
}

}  // namespace

hipError_t launch_rmsnorm_quant(const float* X, const float* G, int64_t M, int64_t K,
                                int8_t* X_q, float* x_scale, int32_t* x_sum, hipStream_t stream) {
  const dim3 grid((unsigned)M);
  const bool wide = K > kQuantWideK;
  const int T = wide ? kQuantWideThreads : kQuantThreads;
  const int64_t per = (K / 4 + T - 1) / T;   // float4 per thread
#define BL_RQ(RR, TT) k_rmsnorm_quant<RR, TT><<<grid, dim3(TT), 0, stream>>>(X, G, K, X_q, x_scale, x_sum)
  if (!wide) {
    if (per <= 1) BL_RQ(1, kQuantThreads);
    else if (per <= 2) BL_RQ(2, kQuantThreads);
    else if (per <= 4) BL_RQ(4, kQuantThreads);
    else if (per <= 8) BL_RQ(8, kQuantThreads);
    else BL_RQ(16, kQuantThreads);
  } else {
    // (16 float4 of row and gain each would spill at 1024 threads' 128 VGPRs)
    if (per <= 4) BL_RQ(4, kQuantWideThreads);
    else if (per <= 8) BL_RQ(8, kQuantWideThreads);
    else BL_RQ(0, kQuantWideThreads);
  }
#undef BL_RQ
  return hipGetLastError();
}

hipError_t launch_quant(const float* X, int64_t M, int64_t K, int8_t* X_q, float* x_scale,
                        int32_t* x_sum, hipStream_t stream, int bits) {
  const float qmax = bits == 4 ? 7.0f : 127.0f;
  const dim3 grid((unsigned)M);
  const bool wide = K > kQuantWideKPlain;
  const int T = wide ? kQuantWideThreads : kQuantThreads;
  const int64_t per = (K / 4 + T - 1) / T;   // float4 per thread
#define BL_Q(RR, TT) k_quant_acts<RR, TT><<<grid, dim3(TT), 0, stream>>>(X, K, X_q, x_scale, x_sum, qmax)
  if (!wide) {
    if (per <= 1) BL_Q(1, kQuantThreads);
    else if (per <= 2) BL_Q(2, kQuantThreads);
    else if (per <= 4) BL_Q(4, kQuantThreads);
    else if (per <= 8) BL_Q(8, kQuantThreads);
    else BL_Q(16, kQuantThreads);
  } else {
    if (per <= 2) BL_Q(2, kQuantWideThreads);
    else if (per <= 4) BL_Q(4, kQuantWideThreads);
    else if (per <= 8) BL_Q(8, kQuantWideThreads);
    else if (per <= 16) BL_Q(16, kQuantWideThreads);
    else BL_Q(0, kQuantWideThreads);   // 32 float4 would spill at 128 VGPRs
  }
#undef BL_Q
  return hipGetLastError();
}

hipError_t launch_quant_multi(int G, const float* const* X, int64_t M, const int64_t* K,
                              int8_t* const* X_q, float* const* x_scale, int32_t* const* x_sum,
                              hipStream_t stream) {
  if (G < 1 || G > kQuantMaxMulti || M < 1) return hipErrorInvalidValue;
  QuantMulti q{};
  int64_t maxK = 0;
  for (int g = 0; g < G; ++g) {
    q.X[g] = X[g]; q.K[g] = K[g]; q.Xq[g] = X_q[g]; q.xs[g] = x_scale[g]; q.xsum[g] = x_sum[g];
    maxK = std::max(maxK, K[g]);
  }
  const dim3 grid((unsigned)(G * M));
  const bool wide = maxK > kQuantWideKPlain;
  const int T = wide ? kQuantWideThreads : kQuantThreads;
  const int64_t per = (maxK / 4 + T - 1) / T;
  const float qmax = 127.0f;
#define BL_QM(RR, TT) k_quant_acts_multi<RR, TT><<<grid, dim3(TT), 0, stream>>>(q, M, qmax)
  if (!wide) {
    if (per <= 1) BL_QM(1, kQuantThreads);
    else if (per <= 2) BL_QM(2, kQuantThreads);
    else if (per <= 4) BL_QM(4, kQuantThreads);
    else if (per <= 8) BL_QM(8, kQuantThreads);
    else BL_QM(16, kQuantThreads);
  } else {
    if (per <= 2) BL_QM(2, kQuantWideThreads);
    else if (per <= 4) BL_QM(4, kQuantWideThreads);
    else if (per <= 8) BL_QM(8, kQuantWideThreads);
    else if (per <= 16) BL_QM(16, kQuantWideThreads);
    else BL_QM(0, kQuantWideThreads);
  }
#undef BL_QM
  return hipGetLastError();
}

}  // namespace bl
