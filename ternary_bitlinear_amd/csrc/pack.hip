// Absmean ternarisation and 2-bit packing of a latent weight matrix.
//
// Page "BitNet b1.58: Mathematical Foundations ..." (llms.blog), section 2,
// "Weight Quantization: Absmean Scaling": gamma = mean |W|, then
// W~ = RoundClip(W / (gamma + eps), -1, 1).
//
// Three launches on the caller's stream:
//   1. k_abs_sum_partials: exact sum of |W| as a fixed-point integer.
//      Every finite fp32 |w| is sig * 2^(eb - 150) (eb = max(exponent field,
//      1)), i.e. an integer number of units of 2^-149.  A wave takes a tile of
//      2048 values, finds the tile's largest exponent and adds the significands
//      shifted to a 35-exponent window into one 64-bit accumulator per lane
//      (32 values < 2^59 each cannot overflow); values below the window (more
//      than 2^35 times smaller than the tile maximum) take an exact slow path.
//      Tile sums go into ten 32-bit "digits" (lane d of the wave holds digit
//      d as a 64-bit counter), so the sum is exact and independent of order.
//   2. k_gamma_finalize: one workgroup adds the per-wave digits, divides the
//      exact integer by N*K and rounds once to fp32 (nearest, ties to even).
//      It also turns the fp32 division-and-round of the quantiser into two
//      fp32 thresholds (see k_gamma_finalize).
//   3. k_ternarize_pack: compares each weight with the thresholds and packs
//      codes W~ + 1 at 2 bits each (format BLT2-v1, described in bitlinear.h).
#include "common.hpp"
#include "kernels.hpp"

namespace bl {

namespace {

constexpr int kAbsThreads = 256;               // 4 waves
constexpr int kAbsWavesPerBlock = kAbsThreads / kWave;
constexpr int kAbsVecPerLane = 8;              // float4 loads per lane per tile
constexpr int kAbsElemsPerLane = 4 * kAbsVecPerLane;
constexpr int kAbsTile = kWave * kAbsElemsPerLane;   // 2048 values per wave tile
constexpr int kAbsWindow = 35;                 // exponent window of the lane accumulator
constexpr int kDigits = 10;                    // 10 x 32 bits cover 2^-149 .. 2^171
constexpr int kMaxAbsBlocks = 2048;

// Bits [32 d, 32 d + 32) of (x << off), for the digit held by lane d.  x < 2^40.
__device__ __forceinline__ uint64_t digit_chunk(uint64_t x, int off, int d) {
  int rel = 32 * d - off;
  if (d >= kDigits || rel >= 64 || rel <= -32) return 0;
  uint64_t v = rel >= 0 ? (x >> rel) : (x << (-rel));
  return v & 0xffffffffull;
}

__global__ __launch_bounds__(kAbsThreads) void k_abs_sum_partials(
    const float4* __restrict__ W4, int64_t n4, int64_t n_tiles, uint64_t* __restrict__ partials) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave_id = (int64_t)blockIdx.x * kAbsWavesPerBlock + (threadIdx.x >> 6);
  const int64_t n_waves = (int64_t)gridDim.x * kAbsWavesPerBlock;
  uint64_t digit = 0;   // lane d < kDigits: digit d (units of 2^(32 d - 149))

  for (int64_t t = wave_id; t < n_tiles; t += n_waves) {
    uint32_t v[kAbsElemsPerLane];
    const int64_t base = t * (kAbsTile / 4);
#pragma unroll
    for (int q = 0; q < kAbsVecPerLane; ++q) {
      const int64_t idx = base + q * kWave + lane;
      float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
      if (idx < n4) f = W4[idx];
      v[4 * q + 0] = abs_bits(f.x);
      v[4 * q + 1] = abs_bits(f.y);
      v[4 * q + 2] = abs_bits(f.z);
      v[4 * q + 3] = abs_bits(f.w);
    }
    // Non-negative floats order like their bit patterns: the largest bit
    // pattern carries the largest exponent.
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < kAbsElemsPerLane; ++i) mx = max(mx, v[i]);
    mx = wave_max_u32(mx);
    const int eb_max = max((int)(mx >> 23), 1);
    const int lb = max(eb_max - kAbsWindow, 1);

    uint64_t acc = 0;
    bool tail = false;
#pragma unroll
    for (int i = 0; i < kAbsElemsPerLane; ++i) {
      const uint32_t e = v[i] >> 23;
      const uint32_t sig = (v[i] & 0x7fffffu) | (min(e, 1u) << 23);
      const int s = max((int)e, 1) - lb;
      const bool in = s >= 0;
      acc += in ? ((uint64_t)sig << (in ? s : 0)) : 0ull;
      tail |= (!in) & (sig != 0);
    }
    // Tile total = acc summed over the wave, < 2^70: sum the 32-bit halves
    // separately (each < 2^38) and place them at bit lb - 1 of the frame.
    const uint64_t lo = wave_sum_u64(acc & 0xffffffffull);
    const uint64_t hi = wave_sum_u64(acc >> 32);
    digit += digit_chunk(lo, lb - 1, lane) + digit_chunk(hi, lb - 1 + 32, lane);

    if (__any(tail)) {
      // Exact slow path for values below the window: one value at a time,
      // broadcast to the digit lanes.
#pragma unroll 1
      for (int i = 0; i < kAbsElemsPerLane; ++i) {
        const uint32_t e = v[i] >> 23;
        const uint32_t sig = (v[i] & 0x7fffffu) | (min(e, 1u) << 23);
        const int eb = max((int)e, 1);
        uint64_t mask = __ballot(eb < lb && sig != 0);
        while (mask) {
          const int src = __ffsll((unsigned long long)mask) - 1;
          const uint32_t s_sig = (uint32_t)__shfl((int)sig, src, kWave);
          const int s_eb = __shfl(eb, src, kWave);
          digit += digit_chunk((uint64_t)s_sig, s_eb - 1, lane);
          mask &= mask - 1;
        }
      }
    }
  }
  if (lane < kDigits) partials[wave_id * kDigits + lane] = digit;
}

// Smallest fp32 >= t.
__device__ __forceinline__ float round_up_f32(double t) {
  float f = (float)t;   // round to nearest
  if ((double)f < t) {
    uint32_t u = __float_as_uint(f);
    if (f > 0.f) u += 1;
    else if (f < 0.f) u -= 1;
    else u = 1u;          // +0 / -0 -> smallest subnormal
    f = __uint_as_float(u);
  }
  return f;
}

// Q * 2^-151 rounded to fp32 (nearest, ties to even); `sticky` says the true
// value exceeds Q * 2^-151 by a positive amount below 2^-151.
__device__ float fixed_to_f32(const uint32_t* Q, int nq, bool sticky) {
  int p = -1;
  for (int i = nq - 1; i >= 0 && p < 0; --i)
    if (Q[i]) p = 32 * i + 31 - __clz(Q[i]);
  if (p < 0) return 0.f;   // value < 2^-151: below half the smallest subnormal
  auto bit = [&](int b) -> uint32_t { return b < 0 ? 0u : (Q[b >> 5] >> (b & 31)) & 1u; };
  const int lsb = max(p - 23, 2);  // Q bit of the significand's last place (2 -> 2^-149)
  uint32_t sig = 0;
  for (int b = p; b >= lsb; --b) sig = (sig << 1) | bit(b);
  const uint32_t round = bit(lsb - 1);
  for (int b = lsb - 2; b >= 0 && !sticky; --b) sticky = bit(b) != 0;
  int l = lsb;
  if (round && (sticky || (sig & 1u))) {
    sig += 1;
    if (sig == (1u << 24)) { sig >>= 1; l += 1; }
  }
  if (sig < (1u << 23)) return __uint_as_float(sig);             // subnormal (l == 2)
  return __uint_as_float(((uint32_t)(l - 1) << 23) | (sig & 0x7fffffu));
}

// One workgroup: total the digits, gamma = RN32(total * 2^-149 / count), and
// the thresholds of the ternary decision.
//
// With g = fp32(gamma + 1e-5) > 0 and z = RN32(w / g):
//   floor(z + 1/2) >= 1  <=>  z >= 1/2  <=>  w / g >= 1/2 - 2^-26
//     (1/2 - 2^-26 is the midpoint below 1/2; the tie rounds to 1/2, whose
//      significand is even)  <=>  w >= g (1/2 - 2^-26);
//   floor(z + 1/2) <= -1 <=>  z < -1/2  <=>  w / g < -(1/2 + 2^-25)
//     (the midpoint above 1/2 rounds to 1/2)  <=>  w < -g (1/2 + 2^-25).
// Both products are exact in fp64 (24-bit times 25-bit significands).  For
// an fp32 w, "w >= t" equals "w >= RU32(t)" and "w < t" equals
// "w < RU32(t)", so two fp32 thresholds decide every weight exactly.
__global__ __launch_bounds__(256) void k_gamma_finalize(const uint64_t* __restrict__ partials,
                                                        int64_t n_partials, int64_t count,
                                                        float* __restrict__ gamma_out,
                                                        float* __restrict__ thresholds) {
  __shared__ uint64_t red[256][kDigits];
  uint64_t d[kDigits];
#pragma unroll
  for (int i = 0; i < kDigits; ++i) d[i] = 0;
  for (int64_t p = threadIdx.x; p < n_partials; p += blockDim.x) {
#pragma unroll
    for (int i = 0; i < kDigits; ++i) d[i] += partials[p * kDigits + i];
  }
#pragma unroll
  for (int i = 0; i < kDigits; ++i) red[threadIdx.x][i] = d[i];
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) {
#pragma unroll
      for (int i = 0; i < kDigits; ++i) red[threadIdx.x][i] += red[threadIdx.x + s][i];
    }
    __syncthreads();
  }
  if (threadIdx.x != 0) return;

  // Normalise to 32-bit digits (S in units of 2^-149), then S4 = 4 S.
  constexpr int kN = kDigits + 2;
  uint32_t S[kN];
  uint64_t carry = 0;
  for (int i = 0; i < kDigits; ++i) {
    const uint64_t t = red[0][i] + carry;
    S[i] = (uint32_t)t;
    carry = t >> 32;
  }
  S[kDigits] = (uint32_t)carry;
  S[kDigits + 1] = (uint32_t)(carry >> 32);
  for (int i = kN - 1; i > 0; --i) S[i] = (S[i] << 2) | (S[i - 1] >> 30);
  S[0] <<= 2;
  // Q = floor(4 S / count) (units of 2^-151), remainder -> sticky.
  uint32_t Q[kN];
  uint64_t rem = 0;
  const uint64_t D = (uint64_t)count;
  for (int i = kN - 1; i >= 0; --i) {
    const uint64_t cur = (rem << 32) | S[i];
    Q[i] = (uint32_t)(cur / D);
    rem = cur % D;
  }
  const float gamma = fixed_to_f32(Q, kN, rem != 0);
  const float g = gamma + 1e-5f;
  gamma_out[0] = gamma;
  thresholds[0] = round_up_f32((double)g * (0.5 - 0x1p-26));
  thresholds[1] = round_up_f32(-(double)g * (0.5 + 0x1p-25));
}

__global__ __launch_bounds__(256) void k_ternarize_pack(const float4* __restrict__ W4,
                                                        int64_t n_words,
                                                        const float* __restrict__ thresholds,
                                                        uint32_t* __restrict__ out) {
  const float t_pos = thresholds[0];
  const float t_neg = thresholds[1];
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t wi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; wi < n_words; wi += stride) {
    float v[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 f = W4[wi * 4 + q];
      v[4 * q + 0] = f.x;
      v[4 * q + 1] = f.y;
      v[4 * q + 2] = f.z;
      v[4 * q + 3] = f.w;
    }
    uint32_t word = 0;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const uint32_t code = v[t] >= t_pos ? 2u : (v[t] < t_neg ? 0u : 1u);
      word |= code << (8 * (t & 3) + 2 * (t >> 2));
    }
    out[wi] = word;
  }
}

// Base-3 packing (BLT3-v1, page section 4 "Memory Bandwidth and Latency
// Bounds": five ternary values per byte).  Thread per 20-weight word of a
// row (rows padded with W~ = 0 to a multiple of 80 weights): the same two
// thresholds decide each code c = W~ + 1, and byte b of the word stores
// Nb = sum_j c_{20g + 4j + b} 3^(4 - j) as ceil(256 Nb / 243).  20 weights
// are five float4 (K % 16 == 0, so a row's last word is cut at a float4).
__global__ __launch_bounds__(256) void k_ternarize_pack3(const float* __restrict__ W, int64_t N,
                                                         int K, const float* __restrict__ thresholds,
                                                         uint32_t* __restrict__ out) {
  const float t_pos = thresholds[0];
  const float t_neg = thresholds[1];
  const int words = 4 * ((K + 79) / 80);
  const int64_t total = N * words;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t n = i / words;
    const int g = (int)(i - n * words);
    uint32_t code[20];
#pragma unroll
    for (int q = 0; q < 5; ++q) {
      const int k = 20 * g + 4 * q;
      float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
      if (k < K) f = *reinterpret_cast<const float4*>(W + n * K + k);
      const float v[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
      for (int t = 0; t < 4; ++t)
        code[4 * q + t] = k >= K ? 1u : (v[t] >= t_pos ? 2u : (v[t] < t_neg ? 0u : 1u));
    }
    uint32_t word = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      uint32_t nb = 0;
#pragma unroll
      for (int j = 0; j < 5; ++j) nb = 3 * nb + code[4 * j + b];
      word |= ((256 * nb + 242) / 243) << (8 * b);
    }
    out[i] = word;
  }
}

int64_t abs_tiles(int64_t nk) { return (nk + kAbsTile - 1) / kAbsTile; }
int64_t abs_blocks(int64_t nk) {
  const int64_t b = (abs_tiles(nk) + kAbsWavesPerBlock - 1) / kAbsWavesPerBlock;
  return b < kMaxAbsBlocks ? b : kMaxAbsBlocks;
}

}  // namespace

size_t pack_workspace_bytes(int64_t N, int64_t K) {
  const int64_t waves = abs_blocks(N * K) * kAbsWavesPerBlock;
  return (size_t)(kPackWsHeader + waves * kDigits * sizeof(uint64_t));
}

hipError_t launch_pack(const float* W, int64_t N, int64_t K, uint8_t* W_packed, float* gamma,
                       void* workspace, hipStream_t stream) {
  const int64_t nk = N * K;
  float* thresholds = reinterpret_cast<float*>(workspace);
  uint64_t* partials =
      reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(workspace) + kPackWsHeader);
  const int64_t blocks = abs_blocks(nk);
  k_abs_sum_partials<<<dim3((unsigned)blocks), dim3(kAbsThreads), 0, stream>>>(
      reinterpret_cast<const float4*>(W), nk / 4, abs_tiles(nk), partials);
  k_gamma_finalize<<<1, 256, 0, stream>>>(partials, blocks * kAbsWavesPerBlock, nk, gamma,
                                          thresholds);
  const int64_t n_words = nk / 16;
  int64_t pb = (n_words + 255) / 256;
  if (pb > 8192) pb = 8192;
  k_ternarize_pack<<<dim3((unsigned)pb), dim3(256), 0, stream>>>(
      reinterpret_cast<const float4*>(W), n_words, thresholds,
      reinterpret_cast<uint32_t*>(W_packed));
  return hipGetLastError();
}

hipError_t launch_pack3(const float* W, int64_t N, int64_t K, uint8_t* W_packed3, float* gamma,
                        void* workspace, hipStream_t stream) {
  const int64_t nk = N * K;
  float* thresholds = reinterpret_cast<float*>(workspace);
  uint64_t* partials =
      reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(workspace) + kPackWsHeader);
  const int64_t blocks = abs_blocks(nk);
  k_abs_sum_partials<<<dim3((unsigned)blocks), dim3(kAbsThreads), 0, stream>>>(
      reinterpret_cast<const float4*>(W), nk / 4, abs_tiles(nk), partials);
  k_gamma_finalize<<<1, 256, 0, stream>>>(partials, blocks * kAbsWavesPerBlock, nk, gamma,
                                          thresholds);
  const int64_t total = N * 4 * ((K + 79) / 80);
  int64_t pb = (total + 255) / 256;
  if (pb > 8192) pb = 8192;
  k_ternarize_pack3<<<dim3((unsigned)pb), dim3(256), 0, stream>>>(
      W, N, (int)K, thresholds, reinterpret_cast<uint32_t*>(W_packed3));
  return hipGetLastError();
}

}  // namespace bl
