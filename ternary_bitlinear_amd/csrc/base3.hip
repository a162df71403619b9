// Base-3 weights (format BLT3-v1): five ternary weights per byte.
//
// Page "BitNet b1.58: Mathematical Foundations ..." (llms.blog), section 4,
// "Memory Bandwidth and Latency Bounds": five ternary values fit one byte
// because 3^5 = 243 < 256, 1.6 bits per weight against the 2 of BLT2-v1.
// Layout (this library's own): code c = W~ + 1; every row is padded with
// W~ = 0 to a multiple of 80 weights (16 bytes); little-endian 32-bit word g
// of a row holds k = 20g + 4j + b (j = 0..4, b = 0..3) in its byte b, which
// stores Nb = sum_j c 3^(4 - j) as ceil(256 Nb / 243).
//
// Decoding: the byte B read as the fraction B / 256 approximates Nb / 243,
// five base-3 digits after the point; B = 3 B moves the next digit into bits
// 8-9 and B & 255 keeps the rest.  Bytes 0 and 2 of a word (and 1 and 3)
// travel together in the 16-bit halves of one register (3 x 255 < 2^10), so
// two multiplies step all four bytes, and digit j of the four bytes lands as
// one int8x4 word: the codes of k = 20g + 4j .. 20g + 4j + 3, in the order
// of four consecutive int8 activations.  Word d = 5g + j of a 16-byte piece
// therefore holds k = 4d .. 4d + 3 of the piece's 80: the decoded piece is 80
// consecutive codes, four words per 16-wide slice of K.
//
// Kernels: k_decode_b3 (one token, v_dot4 on the vector ALU), k_b3_mma (2-16
// tokens, v_mfma_i32_16x16x64_i8 on whole decoded pieces) and k_b3_to_b2 (the
// rewrite to the 2-bit format for the other projection kernels).
#include "common.hpp"
#include "kernels.hpp"

namespace bl {

namespace {

constexpr int kB3Piece = 80;     // weights per 16-byte piece
constexpr int kB3Waves = 4;      // waves per workgroup of the decode kernel

// The five code words of one packed word: c[j] = codes of k = 20g + 4j + 0..3.
__device__ __forceinline__ void decode_b3(uint32_t w, uint32_t (&c)[5]) {
  uint32_t lo = w & 0x00FF00FFu;          // bytes 0 and 2
  uint32_t hi = (w >> 8) & 0x00FF00FFu;   // bytes 1 and 3
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    lo *= 3u;
    hi *= 3u;
    // digit of byte 0 at bits 8-9 of lo, byte 2 at 24-25; bytes 1, 3 in hi
    c[j] = ((lo >> 8) & 0x00FF00FFu) | (hi & 0xFF00FF00u);
    lo &= 0x00FF00FFu;
    hi &= 0x00FF00FFu;
  }
}

struct B3Args {
  const uint8_t* Wp;    // [N][16 * ceil(K / 80)] BLT3-v1
  const float* gamma;
  int N, K, M;
  const int8_t* Xq;     // [M][K]
  const float* xs;      // [M]
  const int32_t* xsum;  // [M]
  void* Y;              // [M][N]
};

// Projection on base-3 weights, 1 <= M <= MT tokens, on the vector ALU.
// Each wave owns R consecutive rows; lane l takes the 16-byte pieces
// p = l + 64 q (80 weights each) of every row, in blocks of Q pieces per
// lane.  The weights of a block are loaded first (all R Q pieces in flight),
// decoded once, and each token's 80 activations per piece are loaded and
// multiplied with v_dot4 (page section 2's integer sum, here on codes
// c = W~ + 1, so the token's sum of activations is subtracted at the end).
// Pieces past the row and 16-weight chunks past K read zero activations.
template <int OUT, int R, int Q, int MT>
__global__ __launch_bounds__(kB3Waves * kWave) void k_decode_b3(B3Args a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = (blockIdx.x * kB3Waves + wave) * R;
  const int N = a.N, K = a.K, M = a.M;
  const int npieces = (K + kB3Piece - 1) / kB3Piece;
  const int64_t rowb = 16 * (int64_t)npieces;
  const float gamma = a.gamma[0];

  int32_t acc[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0;

  for (int p0 = 0; p0 < npieces; p0 += kWave * Q) {
    uint4 wq[R][Q];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint8_t* row = a.Wp + (int64_t)min(n0 + r, N - 1) * rowb;
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int p = p0 + lane + kWave * q;
        wq[r][q] = *reinterpret_cast<const uint4*>(row + 16 * (int64_t)(p < npieces ? p : 0));
      }
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int p = p0 + lane + kWave * q;
      uint32_t cw[R][20];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t w4[4] = {wq[r][q].x, wq[r][q].y, wq[r][q].z, wq[r][q].w};
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          uint32_t c[5];
          decode_b3(w4[g], c);
#pragma unroll
          for (int j = 0; j < 5; ++j) cw[r][5 * g + j] = c[j];
        }
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m >= M) continue;   // uniform; keeps the loop unrollable
        const int8_t* xr = a.Xq + (int64_t)m * K;
        int32_t xw[20];
#pragma unroll
        for (int c = 0; c < 5; ++c) {
          const int k0 = kB3Piece * p + 16 * c;
          const i32x4 v = (p < npieces && k0 < K) ? *reinterpret_cast<const i32x4*>(xr + k0)
                                                  : i32x4{0, 0, 0, 0};
          xw[4 * c + 0] = v.x; xw[4 * c + 1] = v.y; xw[4 * c + 2] = v.z; xw[4 * c + 3] = v.w;
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int t = 0; t < 20; ++t)
            acc[r][m] = __builtin_amdgcn_sdot4((int32_t)cw[r][t], xw[t], acc[r][m], false);
      }
    }
  }
  // Lane r MT + m stores row n0 + r, token m.
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int32_t s = wave_sum_i32(acc[r][m]);
      const int n = n0 + r;
      if (m < M && n < N && lane == r * MT + m)
        store_out<OUT>(a.Y, (int64_t)m * N + n, s - a.xsum[m], gamma, a.xs[m]);
    }
}

// Projection on base-3 weights for 2 <= M <= 16 tokens on the matrix cores
// (v_mfma_i32_16x16x64_i8, activations first, codes second).  A workgroup
// owns RBW blocks of 16 weight rows; its 4 waves split the rows' pieces into
// contiguous ranges, and each wave runs all RBW blocks on every fragment of
// activations it loads.  Lane (j, g) = (lane & 15, lane >> 4) works on row j
// of each block and, per step of 4 pieces, piece 4 m + g: its 80 codes decode
// to 20 code words whose k run consecutively (word d holds k = 4d .. 4d + 3
// of the piece), so slice s (words 4s .. 4s + 3) is the instruction's second
// operand for k = 80 p + 16 s .. + 15, and the lane's first operand is the 16
// activation bytes of token j at the same k.  Each piece is decoded once for
// all tokens.  Pieces are loaded P steps ahead; slices at or past K read zero
// activations (the padding codes then add nothing), as do tokens past M.
// The waves' partial sums are added exactly in LDS; register r of lane
// (j, g) is token 4 g + r of row j.
template <int OUT, int P, int RBW>
__global__ __launch_bounds__(kB3Waves * kWave) void k_b3_mma(B3Args a) {
  __shared__ i32x4 part[kB3Waves - 1][RBW][kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 15, g = lane >> 4;
  const int N = a.N, K = a.K, M = a.M;
  const int npieces = (K + kB3Piece - 1) / kB3Piece;
  const int nsteps = (npieces + 3) / 4;
  const int64_t rowb = 16 * (int64_t)npieces;
  const int nb0 = 16 * RBW * blockIdx.x + j;   // row of this lane in block 0
  const uint8_t* row[RBW];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) row[rb] = a.Wp + (int64_t)min(nb0 + 16 * rb, N - 1) * rowb;
  const int8_t* xr = a.Xq + (int64_t)min(j, M - 1) * K;
  const bool tok = j < M;
  const int m0 = (int)((int64_t)wave * nsteps / kB3Waves);
  const int m1 = (int)((int64_t)(wave + 1) * nsteps / kB3Waves);

  constexpr int NB = P + 1;
  uint4 wq[NB][RBW];
  auto fill = [&](int b, int m) {
    const int p = 4 * min(m, m1 - 1) + g;
    const int64_t off = 16 * (int64_t)(p < npieces ? p : 0);
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) wq[b][rb] = *reinterpret_cast<const uint4*>(row[rb] + off);
  };
  i32x4 acc[RBW];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) acc[rb] = i32x4{0, 0, 0, 0};
  if (m0 < m1) {
#pragma unroll
    for (int b = 0; b < P; ++b) fill(b, m0 + b);
    for (int mb = m0; mb < m1; mb += NB) {
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int m = mb + u;
        if (m >= m1) break;
        fill((u + P) % NB, m + P);
        const int p = 4 * m + g;
        i32x4 xa[5];
#pragma unroll
        for (int sl = 0; sl < 5; ++sl) {
          const int k0 = kB3Piece * p + 16 * sl;
          xa[sl] = (tok && k0 < K) ? *reinterpret_cast<const i32x4*>(xr + k0) : i32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) {
          const uint32_t w4[4] = {wq[u][rb].x, wq[u][rb].y, wq[u][rb].z, wq[u][rb].w};
          uint32_t cw[20];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t c[5];
            decode_b3(w4[q], c);
#pragma unroll
            for (int d = 0; d < 5; ++d) cw[5 * q + d] = c[d];
          }
#pragma unroll
          for (int sl = 0; sl < 5; ++sl) {
            const i32x4 b = {(int32_t)cw[4 * sl], (int32_t)cw[4 * sl + 1], (int32_t)cw[4 * sl + 2],
                             (int32_t)cw[4 * sl + 3]};
            acc[rb] = mfma_i8_16x16x64(xa[sl], b, acc[rb]);
          }
        }
      }
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) part[wave - 1][rb][lane] = acc[rb];
  }
  __syncthreads();
  if (wave > 0) return;
  const float gamma = a.gamma[0];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    const int n = nb0 + 16 * rb;
    if (n >= N) continue;
    i32x4 t = acc[rb];
#pragma unroll
    for (int w = 0; w < kB3Waves - 1; ++w) {
      const i32x4 o = part[w][rb][lane];
      t.x += o.x; t.y += o.y; t.z += o.z; t.w += o.w;
    }
    const int32_t v[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tk = 4 * g + r;
      if (tk < M) store_out<OUT>(a.Y, (int64_t)tk * N + n, v[r] - a.xsum[tk], gamma, a.xs[tk]);
    }
  }
}

template <int OUT, int R, int MT>
hipError_t launch_b3_q(const B3Args& a, hipStream_t stream) {
  static_assert(R * MT <= kWave, "one storing lane per output");
  const int npieces = (a.K + kB3Piece - 1) / kB3Piece;
  const int q = (npieces + kWave - 1) / kWave;   // pieces per lane for the whole row
  const dim3 grid((unsigned)((a.N + R * kB3Waves - 1) / (R * kB3Waves)));
  const dim3 block(kB3Waves * kWave);
  if (q <= 1) k_decode_b3<OUT, R, 1, MT><<<grid, block, 0, stream>>>(a);
  else if (q <= 2) k_decode_b3<OUT, R, 2, MT><<<grid, block, 0, stream>>>(a);
  else if (q <= 3) k_decode_b3<OUT, R, 3, MT><<<grid, block, 0, stream>>>(a);
  else k_decode_b3<OUT, R, 4, MT><<<grid, block, 0, stream>>>(a);   // blocks of 256 pieces
  return hipGetLastError();
}

// One token: the vector-ALU kernel.  Decoding costs about two vector
// instructions per weight, so the rows are spread over more waves: 2 rows per
// wave below 16384 rows (timed on MI355X: 8640 <- 3200 5.8 vs 6.8 us at 4
// rows, 4096 <- 11008 7.6 vs 8.1 us), 4 rows on wider outputs (28672 <- 8192:
// 22.3 vs 22.8 us at 2).
// 2-16 tokens: the matrix-core kernel, which decodes each piece once for all
// tokens (timed against the vector-ALU kernel, same process, identical
// outputs: 28672 <- 8192 at 2 / 8 / 16 tokens 22.1 / 30.6 / 29.9 us against
// 30.2 / 112.7 / 193.2; 4096 <- 11008 9.7 / 10.7 / 11.2 against 9.4 / 21.4 /
// 39.6).  Above 8 tokens the fragments of activations are shared by 4 row
// blocks per wave on outputs of 16384+ rows and by 2 on 8192+ (28672 <- 8192
// at 16 tokens: 29.9 us at 4 blocks, 34.4 at 2, 46.2 at 1; 8192 <- 28672:
// 33.7 at 2, 45.4 at 1, 49.8 at 4); up to 8 tokens one block is fastest.
template <int OUT, int RBW>
hipError_t launch_b3_mma(const B3Args& a, hipStream_t stream) {
  const dim3 grid((unsigned)((a.N + 16 * RBW - 1) / (16 * RBW)));
  k_b3_mma<OUT, 2, RBW><<<grid, dim3(kB3Waves * kWave), 0, stream>>>(a);
  return hipGetLastError();
}

template <int OUT>
hipError_t launch_b3_out(const B3Args& a, hipStream_t stream) {
  if (a.M <= 1) return a.N >= 16384 ? launch_b3_q<OUT, 4, 1>(a, stream)
                                    : launch_b3_q<OUT, 2, 1>(a, stream);
  if (a.M > 8 && a.N >= 16384) return launch_b3_mma<OUT, 4>(a, stream);
  if (a.M > 8 && a.N >= 8192) return launch_b3_mma<OUT, 2>(a, stream);
  return launch_b3_mma<OUT, 1>(a, stream);
}

// BLT3-v1 -> BLT2-v1: thread per (row, piece); the 80 decoded codes of a
// piece are five BLT2 words (16 weights each), word u of the piece collecting
// code words 4u .. 4u + 3 at bit offsets 0, 2, 4, 6 of every byte.
__global__ __launch_bounds__(256) void k_b3_to_b2(const uint8_t* __restrict__ W3, int64_t N,
                                                  int K, uint32_t* __restrict__ W2) {
  const int npieces = (K + kB3Piece - 1) / kB3Piece;
  const int kw = K / 16;
  const int64_t total = N * npieces;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t n = i / npieces;
    const int p = (int)(i - n * npieces);
    const uint4 v = *reinterpret_cast<const uint4*>(W3 + 16 * i);
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
    uint32_t cw[20];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint32_t c[5];
      decode_b3(w4[g], c);
#pragma unroll
      for (int j = 0; j < 5; ++j) cw[5 * g + j] = c[j];
    }
#pragma unroll
    for (int u = 0; u < 5; ++u) {
      const int wi = 5 * p + u;   // BLT2 word of the row
      if (wi < kw)
        W2[n * kw + wi] = cw[4 * u] | (cw[4 * u + 1] << 2) | (cw[4 * u + 2] << 4) | (cw[4 * u + 3] << 6);
    }
  }
}

}  // namespace

size_t packed3_row_bytes(int64_t K) { return (size_t)(16 * ((K + kB3Piece - 1) / kB3Piece)); }

hipError_t launch_forward_b3(const uint8_t* W_packed3, const float* gamma, int64_t N, int64_t K,
                             const int8_t* X_q, const float* x_scale, const int32_t* x_sum,
                             int64_t M, void* Y, int y_dtype, hipStream_t stream) {
  if (M < 1 || M > kBase3MaxTokens) return hipErrorInvalidValue;
  const B3Args a{W_packed3, gamma, (int)N, (int)K, (int)M, X_q, x_scale, x_sum, Y};
  switch (y_dtype) {
    case kOutF32: return launch_b3_out<kOutF32>(a, stream);
    case kOutBF16: return launch_b3_out<kOutBF16>(a, stream);
    default: return launch_b3_out<kOutI32>(a, stream);
  }
}

hipError_t launch_b3_to_b2(const uint8_t* W_packed3, int64_t N, int64_t K, uint8_t* W_packed,
                           hipStream_t stream) {
  const int64_t total = N * ((K + kB3Piece - 1) / kB3Piece);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  k_b3_to_b2<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
      W_packed3, N, (int)K, reinterpret_cast<uint32_t*>(W_packed));
  return hipGetLastError();
}

}  // namespace bl
