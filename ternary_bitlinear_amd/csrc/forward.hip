// The BitLinear projection on packed ternary weights and int8 activations.
//
// Page "BitNet b1.58: Mathematical Foundations ..." (llms.blog), section 2,
// "The Linear Transformation and Rescaling": acc = X~ W~^T in int32, then
// Y = acc * gamma * beta / 127, applied once per output after the integer sum
// (section 6, "Scaling Factor Fusion").
//
// The packed codes are c = W~ + 1 in {0, 1, 2}.  They feed the int8 matrix
// cores unchanged and the kernels subtract sum_k x~_k afterwards:
//   sum_k W~_k x~_k = sum_k c_k x~_k - sum_k x~_k,
// which costs one shift and one mask per four weights to unpack.  Zero padding
// beyond K is harmless because the activation there is zero.
//
// Two kernels, both on v_mfma_i32_16x16x64_i8 (A = activations, tokens as
// rows; B = codes, weight rows as columns):
//   k_decode (M <= 16): one workgroup per 16 weight rows; the K dimension is
//     dealt round-robin to the four waves in groups of four 64-wide chunks
//     (one chunk per lane group), so each lane streams 16-byte pieces of one
//     row; the four waves' partial tiles are added through LDS.  The activation
//     operand is read straight from global memory (L2-resident).
//   k_gemm (M > 16): 128 x 128 output tiles, K in steps of 128, activations and
//     packed codes staged in LDS; codes are expanded in registers.
#include "common.hpp"
#include "kernels.hpp"

namespace bl {

namespace {

constexpr int kOutF32 = 0, kOutBF16 = 1, kOutI32 = 2;

template <int OUT>
__device__ __forceinline__ void store_out(void* Y, int64_t idx, int32_t acc, float gamma,
                                          float scale) {
  if constexpr (OUT == kOutI32) {
    reinterpret_cast<int32_t*>(Y)[idx] = acc;
  } else {
    const float y = ((float)acc * gamma) * scale;
    if constexpr (OUT == kOutF32) reinterpret_cast<float*>(Y)[idx] = y;
    else reinterpret_cast<uint16_t*>(Y)[idx] = f32_to_bf16_rne(y);
  }
}

// Word wi of a packed row, or the all-zero-weights word past the row end.
__device__ __forceinline__ uint32_t load_word(const uint32_t* row, int wi, int kw) {
  return wi < kw ? row[wi] : 0x55555555u;
}

// ---------------------------------------------------------------------------
// Decode: M <= 16 tokens.
// ---------------------------------------------------------------------------
constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / kWave;
constexpr int kDecBatch = 4;                            // chunks loaded ahead per lane

template <bool kAligned64, int OUT>
__global__ __launch_bounds__(kDecThreads) void k_decode(
    const uint8_t* __restrict__ Wp, const float* __restrict__ gamma_p, int N, int K,
    const int8_t* __restrict__ Xq, const float* __restrict__ xs,
    const int32_t* __restrict__ xsum, int M, void* __restrict__ Y) {
  __shared__ i32x4 red[kDecThreads / kWave][kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int j = lane & 15;          // B column (weight row) and A row (token)
  const int g = lane >> 4;          // k group
  const int n0 = blockIdx.x * 16;
  const int kw = K / 16;            // packed words per row
  const int nchunks = (K + 63) / 64;
  const uint32_t* wrow =
      reinterpret_cast<const uint32_t*>(Wp + (int64_t)min(n0 + j, N - 1) * (K / 4));
  const bool tok_ok = j < M;
  const int8_t* xrow = Xq + (int64_t)min(j, M - 1) * K;

  // Chunk group cg covers chunks 4 cg .. 4 cg + 3, one per lane group, so the
  // loop trip count is the same for every lane of a wave (the matrix
  // instructions must run with all lanes active); lanes past the end of K
  // contribute zero activations.
  i32x4 acc = {0, 0, 0, 0};
  for (int cg0 = wave; 4 * cg0 < nchunks; cg0 += kDecWaves * kDecBatch) {
    uint32_t w[kDecBatch][4];
#pragma unroll
    for (int b = 0; b < kDecBatch; ++b) {
      const int c = 4 * (cg0 + b * kDecWaves) + g;
      if (kAligned64) {
        uint4 v = make_uint4(0x55555555u, 0x55555555u, 0x55555555u, 0x55555555u);
        if (c < nchunks) v = *reinterpret_cast<const uint4*>(wrow + 4 * c);
        w[b][0] = v.x; w[b][1] = v.y; w[b][2] = v.z; w[b][3] = v.w;
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) w[b][t] = load_word(wrow, 4 * c + t, kw);
      }
    }
#pragma unroll
    for (int b = 0; b < kDecBatch; ++b) {
      const int c = 4 * (cg0 + b * kDecWaves) + g;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int k = 64 * c + 16 * t;
        i32x4 a = {0, 0, 0, 0};
        if (tok_ok && k < K) a = *reinterpret_cast<const i32x4*>(xrow + k);
        acc = mfma_i8_16x16x64(a, expand_codes(w[b][t]), acc);
      }
    }
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w2 = 1; w2 < kDecThreads / kWave; ++w2) {
    const i32x4 o = red[w2][lane];
    acc.x += o.x; acc.y += o.y; acc.z += o.z; acc.w += o.w;
  }
  const int n = n0 + j;
  if (n >= N) return;
  const float gamma = gamma_p[0];
  const int32_t vals[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 4 * g + r;
    if (m < M) store_out<OUT>(Y, (int64_t)m * N + n, vals[r] - xsum[m], gamma, xs[m]);
  }
}

// ---------------------------------------------------------------------------
// GEMM: M > 16 tokens.
// ---------------------------------------------------------------------------
constexpr int kGemmThreads = 256;
constexpr int kBM = 128, kBN = 128, kBK = 128;
constexpr int kSA = kBK + 16;        // LDS row stride of the activation tile (bytes)
constexpr int kSB = kBK / 4 + 4;     // LDS row stride of the packed code tile (bytes)

template <bool kAligned64, int OUT>
__global__ __launch_bounds__(kGemmThreads) void k_gemm(
    const uint8_t* __restrict__ Wp, const float* __restrict__ gamma_p, int N, int K,
    const int8_t* __restrict__ Xq, const float* __restrict__ xs,
    const int32_t* __restrict__ xsum, int M, void* __restrict__ Y, int tiles_n) {
  __shared__ __attribute__((aligned(16))) int8_t sA[kBM * kSA];
  __shared__ __attribute__((aligned(16))) uint32_t sB[kBN * kSB / 4];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int i = lane & 15, g = lane >> 4;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int kw = K / 16;

  i32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = i32x4{0, 0, 0, 0};

  for (int k0 = 0; k0 < K; k0 += kBK) {
    // activations: 128 rows x 128 bytes, 16-byte pieces
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int chunk = tid + kGemmThreads * q;
      const int r = chunk >> 3, c16 = chunk & 7;
      const int m = m0 + r, k = k0 + 16 * c16;
      i32x4 v = {0, 0, 0, 0};
      if (m < M && k < K) v = *reinterpret_cast<const i32x4*>(Xq + (int64_t)m * K + k);
      *reinterpret_cast<i32x4*>(sA + r * kSA + 16 * c16) = v;
    }
    // codes: 128 rows x 8 words
    {
      const int r = tid >> 1, h = tid & 1;
      const int n = n0 + r;
      const int wi0 = k0 / 16 + 4 * h;
      uint32_t w[4] = {0x55555555u, 0x55555555u, 0x55555555u, 0x55555555u};
      if (n < N) {
        const uint32_t* row = reinterpret_cast<const uint32_t*>(Wp + (int64_t)n * (K / 4));
        if (kAligned64 && wi0 + 4 <= kw) {
          const uint4 v = *reinterpret_cast<const uint4*>(row + wi0);
          w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t) w[t] = load_word(row, wi0 + t, kw);
        }
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) sB[(r * kSB) / 4 + 4 * h + t] = w[t];
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      i32x4 af[4];
      uint32_t bw[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        af[mb] = *reinterpret_cast<const i32x4*>(sA + (wm * 64 + mb * 16 + i) * kSA + ks * 64 +
                                                  g * 16);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) bw[nb] = sB[((wn * 64 + nb * 16 + i) * kSB) / 4 + ks * 4 + g];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const i32x4 bf = expand_codes(bw[nb]);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) acc[mb][nb] = mfma_i8_16x16x64(af[mb], bf, acc[mb][nb]);
      }
    }
    __syncthreads();
  }

  const float gamma = gamma_p[0];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + wm * 64 + mb * 16 + 4 * g + r;
      if (m >= M) continue;
      const int32_t sx = xsum[m];
      const float sc = xs[m];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int n = n0 + wn * 64 + nb * 16 + i;
        if (n < N) store_out<OUT>(Y, (int64_t)m * N + n, acc[mb][nb][r] - sx, gamma, sc);
      }
    }
  }
}

template <bool A64, int OUT>
hipError_t dispatch(const uint8_t* Wp, const float* gamma, int N, int K, const int8_t* Xq,
                    const float* xs, const int32_t* xsum, int M, void* Y, hipStream_t stream) {
  if (M <= 16) {
    const int blocks = (N + 15) / 16;
    k_decode<A64, OUT><<<dim3(blocks), dim3(kDecThreads), 0, stream>>>(Wp, gamma, N, K, Xq, xs,
                                                                       xsum, M, Y);
  } else {
    const int tiles_n = (N + kBN - 1) / kBN;
    const int64_t tiles = (int64_t)tiles_n * ((M + kBM - 1) / kBM);
    k_gemm<A64, OUT><<<dim3((unsigned)tiles), dim3(kGemmThreads), 0, stream>>>(
        Wp, gamma, N, K, Xq, xs, xsum, M, Y, tiles_n);
  }
  return hipGetLastError();
}

template <int OUT>
hipError_t dispatch_out(const uint8_t* Wp, const float* gamma, int N, int K, const int8_t* Xq,
                        const float* xs, const int32_t* xsum, int M, void* Y,
                        hipStream_t stream) {
  if (K % 64 == 0) return dispatch<true, OUT>(Wp, gamma, N, K, Xq, xs, xsum, M, Y, stream);
  return dispatch<false, OUT>(Wp, gamma, N, K, Xq, xs, xsum, M, Y, stream);
}

}  // namespace

hipError_t launch_forward(const uint8_t* W_packed, const float* gamma, int64_t N, int64_t K,
                          const int8_t* X_q, const float* x_scale, const int32_t* x_sum,
                          int64_t M, void* Y, int y_dtype, hipStream_t stream) {
  const int n = (int)N, k = (int)K, m = (int)M;
  switch (y_dtype) {
    case kOutF32:
      return dispatch_out<kOutF32>(W_packed, gamma, n, k, X_q, x_scale, x_sum, m, Y, stream);
    case kOutBF16:
      return dispatch_out<kOutBF16>(W_packed, gamma, n, k, X_q, x_scale, x_sum, m, Y, stream);
    default:
      return dispatch_out<kOutI32>(W_packed, gamma, n, k, X_q, x_scale, x_sum, m, Y, stream);
  }
}

}  // namespace bl
