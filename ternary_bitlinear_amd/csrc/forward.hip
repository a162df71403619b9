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
//   k_decode (M <= 16): a software-pipelined stream over packed rows, see
//     below; the activation operand comes straight from global memory
//     (L2-resident) and is reused across the workgroup's row blocks.
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
//
// K is cut into 64-wide chunks (16 bytes of a packed row) taken four at a time
// ("chunk group", one chunk per lane group g = lane / 16).  For a 16-row block
// a lane loads one 16-byte piece of its row per chunk group and, with the
// matching 64 activations of its token (zero for lanes past M), issues four
// matrix instructions.  Two kernels:
//
// k_decode_lds (activations in LDS).  A workgroup of NW waves owns one 16-row
//   block; the waves split its chunk groups round-robin.  The activations are staged once
//   per workgroup into LDS ([M][K + 16], padded against bank conflicts, plus a
//   16-byte zero slot for lanes past M or K), either copied from X~ (kALds) or
//   quantised from fp32 X in place (kAFuse: each token gets NW / M' waves,
//   M' = M rounded up to a power of two, that hold its row in registers,
//   reduce the absmax and write codes and code sum, with the same per-element
//   arithmetic as the standalone quantiser; workgroup 0 may also write X~,
//   x_scale and x_sum out; the fp32 rows are requested before the weights so
//   they do not queue behind the weight stream).  Weight loads run P chunk
//   groups ahead of the matrix instructions through a ring of registers.  The
//   NW partial tiles are added through LDS at the end.
//
// k_decode_reg (activations from global memory, for M x K beyond LDS).  A
//   workgroup owns RB row blocks; activation fragments, loaded into the ring
//   with the weights, serve all RB blocks.
// ---------------------------------------------------------------------------
constexpr int kAReg = 0, kALds = 1, kAFuse = 2;
constexpr int kLdsBudget = 76 * 1024;   // keeps >= 2 workgroups per CU (160 KB LDS)
constexpr int kFuseMaxVec = 16;      // float4 per thread in the fused prologue

struct DecodeArgs {
  const uint8_t* Wp;
  const float* gamma;
  int N, K, M;
  const int8_t* Xq;        // kAReg / kALds: quantised activations [M][K]
  const float* xs;         //                x_scale [M]
  const int32_t* xsum;     //                x_sum [M]
  const float* X;          // kAFuse: fp32 activations [M][K]
  int8_t* Xq_out;          // kAFuse: optional copies of the quantiser outputs
  float* xs_out;
  int32_t* xsum_out;
  void* Y;
};

// Epilogue of one 16-row block: lane (j, g) holds C[4g + r][j] in vals.
template <int OUT, int AM>
__device__ __forceinline__ void decode_store(const DecodeArgs& da, int n, int g, const i32x4& sum,
                                             const uint32_t* s_wmax, const int32_t* s_wsum,
                                             int gw) {
  if (n >= da.N) return;
  const float gamma = da.gamma[0];
  const int32_t vals[4] = {sum.x, sum.y, sum.z, sum.w};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 4 * g + r;
    if (m >= da.M) continue;
    int32_t sx;
    float sc;
    if constexpr (AM == kAFuse) {
      uint32_t bm = 0;
      sx = 0;
      for (int w2 = 0; w2 < gw; ++w2) {
        bm = max(bm, s_wmax[m * gw + w2]);
        sx += s_wsum[m * gw + w2];
      }
      sc = __uint_as_float(bm) / 127.0f;
    } else {
      sx = da.xsum[m];
      sc = da.xs[m];
    }
    store_out<OUT>(da.Y, (int64_t)m * da.N + n, vals[r] - sx, gamma, sc);
  }
}

__host__ __device__ constexpr int lds_red_bytes(int NW) { return NW * kWave * 16; }
__host__ __device__ constexpr int lds_x_offset(int NW) {
  return lds_red_bytes(NW) + ((2 * NW * 4 + 15) / 16) * 16;
}
inline size_t decode_lds_bytes(int NW, int M, int K) {
  return (size_t)lds_x_offset(NW) + (size_t)M * (K + 16) + 16;
}

template <bool kAligned64, int OUT, int NW, int P, int AM>
__global__ __launch_bounds__(NW * kWave) void k_decode_lds(DecodeArgs da) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  i32x4* red = reinterpret_cast<i32x4*>(smem);                                   // [NW][64]
  uint32_t* s_wmax = reinterpret_cast<uint32_t*>(smem + lds_red_bytes(NW));        // [NW]
  int32_t* s_wsum = reinterpret_cast<int32_t*>(s_wmax + NW);                       // [NW]
  int8_t* xl = reinterpret_cast<int8_t*>(smem + lds_x_offset(NW));               // [M][K+16]
  const int N = da.N, K = da.K, M = da.M;
  const int KP = K + 16;
  int8_t* zero_slot = xl + (int64_t)M * KP;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar math
  const int j = lane & 15;
  const int g = lane >> 4;
  const int kw = K / 16;
  const int nchunks = (K + 63) / 64;
  const int ncg = (nchunks + 3) / 4;
  const int n_it = wave < ncg ? (ncg - wave + NW - 1) / NW : 0;
  const int n0 = 16 * (int)blockIdx.x;
  const uint32_t* wrow =
      reinterpret_cast<const uint32_t*>(da.Wp + (int64_t)min(n0 + j, N - 1) * (K / 4));
  const bool tok_ok = j < M;

  int mp = 1;
  while (mp < M) mp <<= 1;
  const int gw = NW / mp;                    // fused: waves per token (host ensures M <= NW)

  // Fused prologue, part 1: the fp32 activations are requested before the
  // weights so that they do not queue behind the weight stream.
  float4 v[AM == kAFuse ? kFuseMaxVec : 1];
  const int fm = wave / gw;
  const int fGT = gw * kWave;
  const int fgt = (wave - fm * gw) * kWave + lane;
  const bool factive = fm < M;
  if constexpr (AM == kAFuse) {
    const float4* xr = reinterpret_cast<const float4*>(da.X + (int64_t)min(fm, M - 1) * K);
    const int K4 = K / 4;
#pragma unroll
    for (int r = 0; r < kFuseMaxVec; ++r) {
      const int i = fgt + r * fGT;
      v[r] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (factive && i < K4) v[r] = xr[i];
    }
  }

  uint32_t wb[P][4];
  auto fill = [&](int s, int it) {
    const int c = 4 * (wave + NW * it) + g;
    const bool cv = it < n_it && c < nchunks;
    if (kAligned64) {
      uint4 q = make_uint4(0x55555555u, 0x55555555u, 0x55555555u, 0x55555555u);
      if (cv) q = *reinterpret_cast<const uint4*>(wrow + 4 * c);
      wb[s][0] = q.x; wb[s][1] = q.y; wb[s][2] = q.z; wb[s][3] = q.w;
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) wb[s][t] = cv ? load_word(wrow, 4 * c + t, kw) : 0x55555555u;
    }
  };
#pragma unroll
  for (int s = 0; s < P; ++s) fill(s, s);

  if constexpr (AM == kALds) {
    const int per_row = K / 16;
    const int total = M * per_row;
    for (int idx = threadIdx.x; idx < total; idx += NW * kWave) {
      const int m = idx / per_row, q = idx - m * per_row;
      *reinterpret_cast<i32x4*>(xl + (int64_t)m * KP + 16 * q) =
          *reinterpret_cast<const i32x4*>(da.Xq + (int64_t)m * K + 16 * q);
    }
    if (threadIdx.x == 0) *reinterpret_cast<i32x4*>(zero_slot) = i32x4{0, 0, 0, 0};
    __syncthreads();
  } else {
    static_assert(AM == kAFuse, "mode");
    // Part 2: absmax per token, then the codes into LDS.
    const int K4 = K / 4;
    uint32_t lmax = 0;
#pragma unroll
    for (int r = 0; r < kFuseMaxVec; ++r) lmax = max(lmax, absmax4(v[r]));
    lmax = wave_max_u32(lmax);
    if (lane == 0) s_wmax[wave] = lmax;
    __syncthreads();
    uint32_t bmax = 0;
    for (int w2 = 0; w2 < gw; ++w2) bmax = max(bmax, s_wmax[min(fm, mp - 1) * gw + w2]);
    const float inv = 127.0f / (__uint_as_float(bmax) + 1e-5f);
    const bool write_out = blockIdx.x == 0 && da.Xq_out != nullptr;
    int32_t lsum = 0;
#pragma unroll
    for (int r = 0; r < kFuseMaxVec; ++r) {
      const int i = fgt + r * fGT;
      if (factive && i < K4) {
        const uint32_t q = quant4(v[r], inv, lsum);
        *reinterpret_cast<uint32_t*>(xl + (int64_t)fm * KP + 4 * i) = q;
        if (write_out) *reinterpret_cast<uint32_t*>(da.Xq_out + (int64_t)fm * K + 4 * i) = q;
      }
    }
    lsum = wave_sum_i32(lsum);
    if (lane == 0) s_wsum[wave] = lsum;
    if (threadIdx.x == 0) *reinterpret_cast<i32x4*>(zero_slot) = i32x4{0, 0, 0, 0};
    __syncthreads();
    if (write_out && factive && fgt == 0) {
      int32_t t = 0;
      for (int w2 = 0; w2 < gw; ++w2) t += s_wsum[fm * gw + w2];
      da.xsum_out[fm] = t;
      da.xs_out[fm] = __uint_as_float(bmax) / 127.0f;
    }
  }

  // Uniform loop bound and branch: the matrix instructions always run with
  // every lane of the wave active.
  i32x4 acc = {0, 0, 0, 0};
  for (int it0 = 0; it0 < n_it; it0 += P) {
#pragma unroll
    for (int s = 0; s < P; ++s) {
      const int it = it0 + s;
      if (it < n_it) {
        const int c = 4 * (wave + NW * it) + g;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int k = 64 * c + 16 * t;
          const int8_t* src = (tok_ok && c < nchunks && k < K) ? xl + j * KP + k : zero_slot;
          const i32x4 a = *reinterpret_cast<const i32x4*>(src);
          acc = mfma_i8_16x16x64(a, expand_codes(wb[s][t]), acc);
        }
        fill(s, it + P);
      }
    }
  }
  red[wave * kWave + lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  i32x4 sum = red[lane];
#pragma unroll
  for (int w2 = 1; w2 < NW; ++w2) {
    const i32x4 o = red[w2 * kWave + lane];
    sum.x += o.x; sum.y += o.y; sum.z += o.z; sum.w += o.w;
  }
  decode_store<OUT, AM>(da, n0 + j, g, sum, s_wmax, s_wsum, gw);
}

template <bool kAligned64, int OUT, int RB, int NW, int P>
__global__ __launch_bounds__(NW * kWave) void k_decode_reg(DecodeArgs da) {
  static_assert(RB <= NW, "one wave per row block in the epilogue");
  __shared__ i32x4 red[NW * RB * kWave];
  const int N = da.N, K = da.K, M = da.M;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int j = lane & 15;
  const int g = lane >> 4;
  const int rb0 = blockIdx.x * RB;
  const int kw = K / 16;
  const int nchunks = (K + 63) / 64;
  const int ncg = (nchunks + 3) / 4;
  const int n_it = wave < ncg ? (ncg - wave + NW - 1) / NW : 0;   // same for all lanes
  const uint32_t* wrow[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
    wrow[rb] = reinterpret_cast<const uint32_t*>(
        da.Wp + (int64_t)min(16 * (rb0 + rb) + j, N - 1) * (K / 4));
  const bool tok_ok = j < M;
  const int8_t* xrow = da.Xq + (int64_t)min(j, M - 1) * K;

  uint32_t wb[P][RB][4];
  i32x4 ab[P][4];
  auto fill = [&](int s, int it) {
    const int c = 4 * (wave + NW * it) + g;
    const bool cv = it < n_it && c < nchunks;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (kAligned64) {
        uint4 v = make_uint4(0x55555555u, 0x55555555u, 0x55555555u, 0x55555555u);
        if (cv) v = *reinterpret_cast<const uint4*>(wrow[rb] + 4 * c);
        wb[s][rb][0] = v.x; wb[s][rb][1] = v.y; wb[s][rb][2] = v.z; wb[s][rb][3] = v.w;
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t)
          wb[s][rb][t] = cv ? load_word(wrow[rb], 4 * c + t, kw) : 0x55555555u;
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int k = 64 * c + 16 * t;
      i32x4 a = {0, 0, 0, 0};
      if (cv && tok_ok && k < K) a = *reinterpret_cast<const i32x4*>(xrow + k);
      ab[s][t] = a;
    }
  };

  i32x4 acc[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) acc[rb] = i32x4{0, 0, 0, 0};
#pragma unroll
  for (int s = 0; s < P; ++s) fill(s, s);
  for (int it0 = 0; it0 < n_it; it0 += P) {
#pragma unroll
    for (int s = 0; s < P; ++s) {
      if (it0 + s < n_it) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            acc[rb] = mfma_i8_16x16x64(ab[s][t], expand_codes(wb[s][rb][t]), acc[rb]);
        }
        fill(s, it0 + s + P);
      }
    }
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) red[(wave * RB + rb) * kWave + lane] = acc[rb];
  __syncthreads();
  if (wave >= RB) return;
  const int rb = wave;
  i32x4 sum = red[rb * kWave + lane];
#pragma unroll
  for (int w2 = 1; w2 < NW; ++w2) {
    const i32x4 o = red[(w2 * RB + rb) * kWave + lane];
    sum.x += o.x; sum.y += o.y; sum.z += o.z; sum.w += o.w;
  }
  decode_store<OUT, kAReg>(da, 16 * (rb0 + rb) + j, g, sum, nullptr, nullptr, 0);
}

// Launch geometry of the decode kernels for one shape.
struct DecodeCfg {
  int am;       // kAReg, kALds, kAFuse; -1: the fused kernel cannot take the shape
  int nw, p;    // waves per workgroup, ring depth
  int rb;       // kAReg: row blocks per workgroup
  int grid;     // workgroups
};

// The choices below come from timing sweeps on MI355X over the decode shapes
// (3B, 7B and 70B projections, M = 1, 8, 16), with the weights cold in HBM.
inline DecodeCfg decode_cfg(int M, int N, int K, bool fused) {
  DecodeCfg c{};
  const int nrb = (N + 15) / 16;
  const int ncg = ((K + 63) / 64 + 3) / 4;
  int mp = 1;
  while (mp < M) mp <<= 1;
  int nw = nrb >= 1024 ? 4 : 8;
  while (nw > 1 && nw > ncg) nw >>= 1;
  const bool lds_ok = decode_lds_bytes(nw, M, K) <= (size_t)kLdsBudget;
  if (fused) {
    // Every workgroup re-quantises the fp32 rows it needs; that redundant
    // read pays for itself only while the workgroups are few.
    const bool regs = mp <= nw && (K / 4 + (nw / mp) * kWave - 1) / ((nw / mp) * kWave) <= kFuseMaxVec;
    c.am = lds_ok && regs && nrb <= 512 ? kAFuse : -1;
  } else {
    c.am = lds_ok ? kALds : kAReg;
  }
  if (c.am == kAFuse || c.am == kALds) {
    c.nw = nw;
    c.p = 2;
    c.grid = nrb;       // one 16-row block per workgroup
    c.rb = 1;
  } else if (c.am == kAReg) {
    // Row blocks sharing each activation fragment: as many as keep >= 224
    // workgroups.
    c.rb = 8;
    while (c.rb > 1 && nrb / c.rb < 224) c.rb /= 2;
    if (M <= 4) c.rb = 1;
    if (c.rb == 8) { c.nw = 8; c.p = 2; }
    else if (c.rb == 4) { c.nw = 4; c.p = 2; }
    else { c.nw = 8; c.p = 4; }
    c.grid = (nrb + c.rb - 1) / c.rb;
  }
  return c;
}

template <bool A64, int OUT, int NW, int AM>
hipError_t launch_decode_lds_t(const DecodeCfg& c, const DecodeArgs& da, hipStream_t stream) {
  const size_t lds = decode_lds_bytes(NW, da.M, da.K);
  auto kern = k_decode_lds<A64, OUT, NW, 2, AM>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  kern<<<dim3(c.grid), dim3(NW * kWave), lds, stream>>>(da);
  return hipGetLastError();
}

template <bool A64, int OUT, int RB, int NW, int P>
hipError_t launch_decode_reg_t(const DecodeCfg& c, const DecodeArgs& da, hipStream_t stream) {
  k_decode_reg<A64, OUT, RB, NW, P><<<dim3(c.grid), dim3(NW * kWave), 0, stream>>>(da);
  return hipGetLastError();
}

template <bool A64, int OUT>
hipError_t launch_decode(const DecodeCfg& c, const DecodeArgs& da, hipStream_t stream) {
  if (c.am == kALds || c.am == kAFuse) {
#define BL_DL(NW)                                                                          \
  if (c.nw == NW)                                                                          \
    return c.am == kALds ? launch_decode_lds_t<A64, OUT, NW, kALds>(c, da, stream)         \
                         : launch_decode_lds_t<A64, OUT, NW, kAFuse>(c, da, stream);
    BL_DL(8) BL_DL(4) BL_DL(2) BL_DL(1)
#undef BL_DL
  } else if (c.am == kAReg) {
#define BL_DR(RB, NW, P) \
  if (c.rb == RB && c.nw == NW && c.p == P) return launch_decode_reg_t<A64, OUT, RB, NW, P>(c, da, stream);
    BL_DR(1, 8, 4) BL_DR(2, 8, 4) BL_DR(4, 4, 2) BL_DR(8, 8, 2)
#undef BL_DR
  }
  return hipErrorInvalidValue;
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
    DecodeArgs da{Wp, gamma, N, K, M, Xq, xs, xsum, nullptr, nullptr, nullptr, nullptr, Y};
    return launch_decode<A64, OUT>(decode_cfg(M, N, K, false), da, stream);
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

namespace bl {

size_t forward_f32_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 16 && decode_cfg((int)M, (int)N, (int)K, true).am == kAFuse) return 0;
  return (size_t)(((M * K + 255) / 256) * 256 + ((8 * M + 255) / 256) * 256);
}

namespace {
template <int OUT>
hipError_t fused_out(const DecodeCfg& c, const DecodeArgs& da, hipStream_t stream) {
  if (da.K % 64 == 0) return launch_decode<true, OUT>(c, da, stream);
  return launch_decode<false, OUT>(c, da, stream);
}
}  // namespace

hipError_t launch_forward_f32(const uint8_t* W_packed, const float* gamma, int64_t N, int64_t K,
                              const float* X, int64_t M, void* Y, int y_dtype, int8_t* X_q_out,
                              float* x_scale_out, int32_t* x_sum_out, void* workspace,
                              hipStream_t stream) {
  const int n = (int)N, k = (int)K, m = (int)M;
  if (M <= 16) {
    const DecodeCfg c = decode_cfg(m, n, k, true);
    if (c.am == kAFuse) {
      DecodeArgs da{W_packed, gamma, n, k, m, nullptr, nullptr, nullptr, X,
                    X_q_out, x_scale_out, x_sum_out, Y};
      switch (y_dtype) {
        case kOutF32: return fused_out<kOutF32>(c, da, stream);
        case kOutBF16: return fused_out<kOutBF16>(c, da, stream);
        default: return fused_out<kOutI32>(c, da, stream);
      }
    }
  }
  // Two launches: quantise into the caller's output buffers (or the
  // workspace), then the projection.
  int8_t* xq = X_q_out;
  float* xs = x_scale_out;
  int32_t* xsum = x_sum_out;
  if (xq == nullptr) {
    char* w = reinterpret_cast<char*>(workspace);
    xq = reinterpret_cast<int8_t*>(w);
    xs = reinterpret_cast<float*>(w + ((M * K + 255) / 256) * 256);
    xsum = reinterpret_cast<int32_t*>(xs + M);
  }
  hipError_t e = launch_quant(X, M, K, xq, xs, xsum, stream);
  if (e != hipSuccess) return e;
  return launch_forward(W_packed, gamma, N, K, xq, xs, xsum, M, Y, y_dtype, stream);
}

}  // namespace bl
