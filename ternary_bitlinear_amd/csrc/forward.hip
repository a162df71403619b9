// The BitLinear projection on packed ternary weights and int8 activations.
//
// Page "BitNet b1.58: Mathematical Foundations ..." (llms.blog), section 2,
// "The Linear Transformation and Rescaling": acc = X~ W~^T in int32, then
// Y = acc * gamma * beta / 127, applied once per output after the integer sum
// (section 6, "Scaling Factor Fusion").
//
// The packed codes are c = W~ + 1 in {0, 1, 2}.  They feed the int8 dot
// products unchanged and sum_k x~_k removes the offset afterwards:
//   sum_k W~_k x~_k = sum_k c_k x~_k - sum_k x~_k,
// which costs shifts and masks only (7 vector instructions per 16 weights)
// to unpack.  Zero padding beyond K is harmless because the activation there
// is zero.
//
// Kernels, by token count M (the host-side rule is in the dispatchers below):
//   k_decode_dot (M = 1, rows up to 4096 values, and the fused single-token
//     calls): v_dot4 on the 2-bit code fields masked in registers, the
//     quantiser optionally in the prologue;
//   k_decode (M <= 16): v_mfma_i32_16x16x64_i8, activations first, a
//     software-pipelined stream over packed rows;
//   k_skinny (2 <= M <= 64, K % 64 == 0): the same instruction over an LDS
//     ring of activations and codes, with an optional K split;
//   k_gemm (M > 16 where k_skinny does not apply): v_mfma_i32_32x32x32_i8,
//     activations first, 64 x 64 / 128 x 128 / 128 x 256 tiles, K in steps
//     of 128 through a 3- or 4-stage LDS ring of direct loads; split-K with
//     k_splitk_reduce when there are few tiles;
//   k_stream (stream.hpp, M = 1): several projections in one persistent
//     launch.
#include "common.hpp"
#include "kernels.hpp"
#include "stream.hpp"

#include <algorithm>
#include <atomic>

namespace bl {

namespace {

// Four consecutive outputs Y[idx .. idx + 3] (idx a multiple of 4, Y aligned
// for the vector), one store.
template <int OUT>
__device__ __forceinline__ void store_out4(void* Y, int64_t idx, i32x4 acc, float gamma,
                                           float scale) {
  if constexpr (OUT == kOutI32) {
    *reinterpret_cast<i32x4*>(reinterpret_cast<int32_t*>(Y) + idx) = acc;
  } else {
    float y[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) y[j] = ((float)acc[j] * gamma) * scale;
    if constexpr (OUT == kOutF32) {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(Y) + idx) = make_float4(y[0], y[1], y[2], y[3]);
    } else {
      const uint32_t lo = (uint32_t)f32_to_bf16_rne(y[0]) | ((uint32_t)f32_to_bf16_rne(y[1]) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16_rne(y[2]) | ((uint32_t)f32_to_bf16_rne(y[3]) << 16);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(Y) + idx) = make_uint2(lo, hi);
    }
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
constexpr int kLdsBudgetFew = 144 * 1024;   // one workgroup per CU
constexpr int kFuseMaxVec = 16;      // float4 per thread in the fused prologue

constexpr int kMaxGroup = kMaxGroupProjections;   // projections of one activation matrix per launch

struct DecodeArgs {
  // Projections sharing the activations (G = 1 for a single one): packed
  // weights, gamma, rows and output of projection g, and the first work unit
  // (workgroup or wave, as the kernel counts them) that serves it.
  const uint8_t* Wp[kMaxGroup];
  const float* gamma[kMaxGroup];
  int Ng[kMaxGroup];
  void* Y[kMaxGroup];
  int first[kMaxGroup + 1];
  int G;
  int K, M;
  const int8_t* Xq;        // kAReg / kALds: quantised activations [M][K]
  const float* xs;         //                x_scale [M]
  const int32_t* xsum;     //                x_sum [M]
  const float* X;          // kAFuse: fp32 activations [M][K]
  const float* norm_g;     // fused single-token decode with RMS normalisation: gain [K]
  int8_t* Xq_out;          // kAFuse: optional copies of the quantiser outputs
  float* xs_out;
  int32_t* xsum_out;
  int splits;              // k_skinny, one projection: K splits (<= 1: none)
  int32_t* part;           //   and their raw partial accumulators [splits][M][N]
};

inline DecodeArgs decode_args_one(const uint8_t* Wp, const float* gamma, int N, int K, int M,
                                  void* Y) {
  DecodeArgs da{};
  da.Wp[0] = Wp;
  da.gamma[0] = gamma;
  da.Ng[0] = N;
  da.Y[0] = Y;
  da.G = 1;
  da.K = K;
  da.M = M;
  return da;
}

// Work units per projection: first[g] = sum over g' < g of ceil(N_g' / rows).
inline int set_units(DecodeArgs& da, int rows_per_unit) {
  da.first[0] = 0;
  for (int g = 0; g < kMaxGroup; ++g)
    da.first[g + 1] = da.first[g] + (g < da.G ? (da.Ng[g] + rows_per_unit - 1) / rows_per_unit : 0);
  return da.first[da.G];
}

// Rows of all projections, each rounded up to whole 16-row blocks (sizes the
// launch geometry of a grouped launch as one matrix of that many rows).
inline int decode_rows(const DecodeArgs& da) {
  int n = 0;
  for (int g = 0; g < da.G; ++g) n += 16 * ((da.Ng[g] + 15) / 16);
  return n;
}

// The projection a work unit serves, and the unit's index within it.  The
// fields are picked with constant indices (no dynamic indexing of the
// kernel arguments); `unit` is uniform over the wave.
struct DecodeView {
  const uint8_t* Wp;
  const float* gamma;
  int N;
  void* Y;
  int unit;
};

// Branch-free: every entry is read at once and picked by selects, so the
// (scalar) argument loads issue together instead of as a chain of
// load-wait-branch steps ahead of the first weight load.
__device__ __forceinline__ DecodeView decode_view(const DecodeArgs& da, int unit) {
  int g = 0;
#pragma unroll
  for (int i = 1; i < kMaxGroup; ++i) g += (i < da.G && unit >= da.first[i]) ? 1 : 0;
  DecodeView v{da.Wp[0], da.gamma[0], da.Ng[0], da.Y[0], unit - da.first[0]};
#pragma unroll
  for (int i = 1; i < kMaxGroup; ++i) {
    const bool pick = g == i;
    v.Wp = pick ? da.Wp[i] : v.Wp;
    v.gamma = pick ? da.gamma[i] : v.gamma;
    v.N = pick ? da.Ng[i] : v.N;
    v.Y = pick ? da.Y[i] : v.Y;
    v.unit = pick ? unit - da.first[i] : v.unit;
  }
  return v;
}

// Per-token epilogue inputs of lane group g (tokens 4g .. 4g + 3), read when
// the kernel starts so that no memory round trip follows the reduction.
struct DecodeEpi {
  float gamma;
  int32_t sx[4];
  float sc[4];
};

__device__ __forceinline__ DecodeEpi decode_epi_load(const DecodeArgs& da, const DecodeView& v,
                                                    int g) {
  DecodeEpi e;
  e.gamma = v.gamma[0];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = min(4 * g + r, da.M - 1);
    e.sx[r] = da.xsum[m];
    e.sc[r] = da.xs[m];
  }
  return e;
}

// Fused mode: the token sums and scales come from the prologue's LDS
// partials (gw waves per token).
__device__ __forceinline__ void decode_epi_fused(DecodeEpi& e, int g, int M,
                                                 const uint32_t* s_wmax, const int32_t* s_wsum,
                                                 int gw) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = min(4 * g + r, M - 1);
    uint32_t bm = 0;
    int32_t sum = 0;
    for (int w2 = 0; w2 < gw; ++w2) {
      bm = max(bm, s_wmax[m * gw + w2]);
      sum += s_wsum[m * gw + w2];
    }
    e.sx[r] = sum;
    e.sc[r] = __uint_as_float(bm) / 127.0f;
  }
}

// Epilogue of one 16-row block: lane (j, g) holds C[4g + r][j] in sum.
template <int OUT>
__device__ __forceinline__ void decode_store(const DecodeView& v, int M, int n, int g,
                                             const i32x4& sum, const DecodeEpi& e) {
  if (n >= v.N) return;
  const int32_t vals[4] = {sum.x, sum.y, sum.z, sum.w};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 4 * g + r;
    if (m < M) store_out<OUT>(v.Y, (int64_t)m * v.N + n, vals[r] - e.sx[r], e.gamma, e.sc[r]);
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
  const DecodeView view = decode_view(da, blockIdx.x);
  const int N = view.N, K = da.K, M = da.M;
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
  const int n0 = 16 * view.unit;
  const uint32_t* wrow =
      reinterpret_cast<const uint32_t*>(view.Wp + (int64_t)min(n0 + j, N - 1) * (K / 4));
  const bool tok_ok = j < M;

  int mp = 1;
  while (mp < M) mp <<= 1;
  const int gw = NW / mp;                    // fused: waves per token (host ensures M <= NW)

  DecodeEpi epi;
  if constexpr (AM == kAFuse) epi.gamma = view.gamma[0];
  else epi = decode_epi_load(da, view, g);

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
      // Plain loads: with the non-temporal hint this kernel measured 7-11 %
      // slower at K = 8192 and 28672 (one token).
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
  if constexpr (AM == kAFuse) decode_epi_fused(epi, g, M, s_wmax, s_wsum, gw);
  decode_store<OUT>(view, M, n0 + j, g, sum, epi);
}

template <bool kAligned64, int OUT, int RB, int NW, int P>
__global__ __launch_bounds__(NW * kWave) void k_decode_reg(DecodeArgs da) {
  static_assert(RB <= NW, "one wave per row block in the epilogue");
  __shared__ i32x4 red[NW * RB * kWave];
  const DecodeView view = decode_view(da, blockIdx.x);
  const int N = view.N, K = da.K, M = da.M;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int j = lane & 15;
  const int g = lane >> 4;
  const int rb0 = view.unit * RB;
  const int kw = K / 16;
  const int nchunks = (K + 63) / 64;
  const int ncg = (nchunks + 3) / 4;
  const int n_it = wave < ncg ? (ncg - wave + NW - 1) / NW : 0;   // same for all lanes
  const uint32_t* wrow[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
    wrow[rb] = reinterpret_cast<const uint32_t*>(
        view.Wp + (int64_t)min(16 * (rb0 + rb) + j, N - 1) * (K / 4));
  const bool tok_ok = j < M;
  const int8_t* xrow = da.Xq + (int64_t)min(j, M - 1) * K;
  const DecodeEpi epi = decode_epi_load(da, view, g);

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
  decode_store<OUT>(view, M, 16 * (rb0 + rb) + j, g, sum, epi);
}

// Launch geometry of the decode kernels for one shape.
struct DecodeCfg {
  int am;       // kAReg, kALds, kAFuse; -1: the fused kernel cannot take the shape
  int nw, p;    // waves per workgroup, ring depth
  int rb;       // kAReg: row blocks per workgroup
  int grid;     // workgroups
};

// The choices below come from timing sweeps on MI355X over the decode shapes
// (3B, 7B and 70B projections, M = 1, 8, 16), with the weights cold in HBM:
//  - at most 256 row blocks (no more workgroups than CUs): 16 waves per
//    workgroup, and the activations may take most of the LDS (one workgroup
//    per CU is all these shapes run anyway);
//  - 257..512 row blocks with long rows: a ring of 4 chunk groups;
//  - 1024 row blocks or more: 4 waves.
inline DecodeCfg decode_cfg(int M, int N, int K, bool fused) {
  DecodeCfg c{};
  const int nrb = (N + 15) / 16;
  const int ncg = ((K + 63) / 64 + 3) / 4;
  int mp = 1;
  while (mp < M) mp <<= 1;
  int nw = nrb >= 1024 ? 4 : (nrb <= 256 ? 16 : 8);
  while (nw > 1 && nw > ncg) nw >>= 1;
  const size_t budget = nrb <= 256 ? kLdsBudgetFew : (size_t)kLdsBudget;
  const bool lds_ok = decode_lds_bytes(nw, M, K) <= budget;
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
    c.p = (nw == 8 && nrb > 256 && nrb <= 512 && ncg >= 8 * nw) ? 4 : 2;
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

template <bool A64, int OUT, int NW, int P, int AM>
hipError_t launch_decode_lds_t(const DecodeCfg& c, DecodeArgs da, hipStream_t stream) {
  (void)c;
  const int grid = set_units(da, 16);   // one 16-row block per workgroup
  const size_t lds = decode_lds_bytes(NW, da.M, da.K);
  auto kern = k_decode_lds<A64, OUT, NW, P, AM>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  kern<<<dim3(grid), dim3(NW * kWave), lds, stream>>>(da);
  return hipGetLastError();
}

template <bool A64, int OUT, int RB, int NW, int P>
hipError_t launch_decode_reg_t(const DecodeCfg& c, DecodeArgs da, hipStream_t stream) {
  (void)c;
  const int grid = set_units(da, 16 * RB);
  k_decode_reg<A64, OUT, RB, NW, P><<<dim3(grid), dim3(NW * kWave), 0, stream>>>(da);
  return hipGetLastError();
}

template <bool A64, int OUT>
hipError_t launch_decode(const DecodeCfg& c, const DecodeArgs& da, hipStream_t stream) {
  if (c.am == kALds || c.am == kAFuse) {
#define BL_DL(NW, P)                                                                       \
  if (c.nw == NW && c.p == P)                                                              \
    return c.am == kALds ? launch_decode_lds_t<A64, OUT, NW, P, kALds>(c, da, stream)      \
                         : launch_decode_lds_t<A64, OUT, NW, P, kAFuse>(c, da, stream);
    BL_DL(16, 2) BL_DL(8, 2) BL_DL(8, 4) BL_DL(4, 2) BL_DL(2, 2) BL_DL(1, 2)
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
// Single-token decode on the vector ALU (M = 1, K % 64 == 0).
//
// Each wave owns R consecutive rows.  Lane l takes the 16-byte pieces
// p = l, l + 64, ... (Q of them; 64 weights each) of a row, so the wave's
// loads of one row are contiguous and whole cache lines.  The lane's 64
// activations per piece are loaded once into registers and serve all R
// rows.  Each 2-bit field of the code bytes is masked in place and
// multiplied with v_dot4_i32_i8 (four products per instruction, one
// accumulator per field: dot_word_fields); a wave shuffle sums each row.  At
// one token the matrix instruction would compute 16 columns to keep one.  Lanes past a row's end re-read its first piece and
// multiply it by zeroed activations.
//
// FUSE = kDotFuseBlock (fp32 input) quantises the token inside the kernel,
// with the same per-element arithmetic as the standalone quantiser (absmax on
// bit patterns, one correctly rounded divide, one multiply and the exact
// round-half-up per element).  The WV waves of a workgroup convert the row
// once: each thread takes every (64 WV)-th group of four, the absmax and the
// code sum go through LDS (two barriers), and each lane then reads its
// piece's codes from LDS.  (Every wave converting the whole row itself, with
// wave reductions only, measured 35-45 % slower: the conversion is then
// repeated per wave.)  The weight loads are issued before the quantiser's
// chain starts, and workgroup 0 may also write X~, x_scale and x_sum out.
// ---------------------------------------------------------------------------
constexpr int kDotFuseNone = 0, kDotFuseBlock = 1;
constexpr int kDotHeldQ = 3;   // pieces per lane whose activations stay in registers
constexpr int kDotWaves = 4;   // waves per workgroup without block fusion

template <int OUT, int R, int Q, int FUSE, int WV, bool NORM = false>
__global__ __launch_bounds__(WV * kWave) void k_decode_dot(DecodeArgs da) {
  static_assert(!NORM || FUSE == kDotFuseBlock, "normalisation only in the block-fused prologue");
  constexpr int kFuseK4 = 64 * 64 / 4 * Q;                   // groups of four at K = 4096 Q
  constexpr int kJ = FUSE == kDotFuseBlock ? kFuseK4 / (WV * kWave) : 1;   // groups per thread
  __shared__ uint32_t s_codes[FUSE == kDotFuseBlock ? kFuseK4 : 1];
  __shared__ uint32_t s_red[2][WV];
  __shared__ SqShared<WV * kWave> s_sq[1];   // used with NORM only
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int unit = blockIdx.x * WV + wave;   // the wave's index over all projections
  const DecodeView view = decode_view(da, unit);
  const int N = view.N, K = da.K;
  const int npieces = K / 64;
  // A wave past the last projection's rows (fewer than WV of them) reads
  // that projection's last row and stores nothing; no early exit, so the
  // argument loads issue as one batch (and every wave reaches the barriers).
  const int n0 = view.unit * R;

  uint4 wq[R][Q];
  auto load_weights = [&]() {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint8_t* row = view.Wp + (int64_t)min(n0 + r, N - 1) * (K / 4);
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int p = lane + kWave * q;
        wq[r][q] = load_once16(row + 16 * (p < npieces ? p : 0));
      }
    }
  };
  // Unfused: weights first (the long-latency stream), then the activations.
  // Fused: the fp32 activations first, then the weights, then the
  // quantiser's chain (reduce, convert, reduce).  Loads complete in issue
  // order, so activations requested after the weights could not be used
  // before the weights had arrived; the scheduling barriers keep the
  // compiler from sinking the weight loads below the chain.
  // The epilogue's gamma and output pointer are read after the weight loads
  // are issued: a wait for their scalar loads (one of them a global one)
  // must not hold up the weight stream.
  float gamma;
  void* yout;
  if constexpr (FUSE == kDotFuseNone) {
    load_weights();
    gamma = view.gamma[0];
    yout = view.Y;
  }
  int32_t xa[Q][16];
  int32_t sx;
  float sc;
  if constexpr (FUSE == kDotFuseBlock) {
    const int K4 = K / 4;
    const float4* src = reinterpret_cast<const float4*>(da.X);
    float4 xv[kJ];
    float4 gv[NORM ? kJ : 1];
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int i = threadIdx.x + WV * kWave * j;
      xv[j] = src[i < K4 ? i : 0];
      if constexpr (NORM) gv[j] = reinterpret_cast<const float4*>(da.norm_g)[i < K4 ? i : 0];
    }
    __builtin_amdgcn_sched_barrier(0);
    load_weights();
    __builtin_amdgcn_sched_barrier(0);
    gamma = view.gamma[0];
    yout = view.Y;
    asm volatile("" ::"s"(gamma), "s"(yout));
    if constexpr (NORM) {
      // RMS normalisation first: the standalone normalising quantiser's
      // arithmetic (an exact mean of squares rounded once, so the partition
      // of the row does not matter).  Groups past the row's end were loaded
      // from its first group and are skipped.
      auto visit = [&](auto&& f) {
#pragma unroll
        for (int j = 0; j < kJ; ++j)
          if (threadIdx.x + WV * kWave * j < K4) f(xv[j]);
      };
      float ms;
      if (!block_mean_square_fast<WV * kWave>(visit, (uint32_t)K, s_sq[0], ms)) {
        ms = block_mean_square_exact<WV * kWave>(src, K4, (uint32_t)K, s_sq[0]);
#pragma unroll
        for (int j = 0; j < kJ; ++j) {   // reloaded: nothing held across the exact path
          const int i = threadIdx.x + WV * kWave * j;
          xv[j] = src[i < K4 ? i : 0];
          gv[j] = reinterpret_cast<const float4*>(da.norm_g)[i < K4 ? i : 0];
        }
      }
      const float rr = rms_reciprocal(ms);
#pragma unroll
      for (int j = 0; j < kJ; ++j) xv[j] = rms_apply(xv[j], rr, gv[j]);
    }
    uint32_t lmax = 0;
#pragma unroll
    for (int j = 0; j < kJ; ++j)
      if (threadIdx.x + WV * kWave * j < K4) lmax = max(lmax, absmax4(xv[j]));
    lmax = wave_max_u32(lmax);
    if (lane == 0) s_red[0][wave] = lmax;
    __syncthreads();
    uint32_t bmax = s_red[0][0];
#pragma unroll
    for (int w = 1; w < WV; ++w) bmax = max(bmax, s_red[0][w]);
    const float beta = __uint_as_float(bmax);
    const float inv = 127.0f / (beta + 1e-5f);
    const bool write_out = blockIdx.x == 0 && da.Xq_out != nullptr;
    int32_t lsum = 0;
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int i = threadIdx.x + WV * kWave * j;
      if (i < K4) {
        const uint32_t c = quant4(xv[j], inv, lsum);
        s_codes[i] = c;
        if (write_out) reinterpret_cast<uint32_t*>(da.Xq_out)[i] = c;
      }
    }
    lsum = wave_sum_i32(lsum);
    if (lane == 0) s_red[1][wave] = (uint32_t)lsum;
    __syncthreads();
    int32_t tsum = 0;
#pragma unroll
    for (int w = 0; w < WV; ++w) tsum += (int32_t)s_red[1][w];
    sx = tsum;
    sc = beta / 127.0f;
    if (write_out && threadIdx.x == 0) {
      da.xs_out[0] = sc;
      da.xsum_out[0] = sx;
    }
#pragma unroll
    for (int q = 0; q < (Q <= kDotHeldQ ? Q : 0); ++q) {
      const int p = lane + kWave * q;
      const i32x4* lp = reinterpret_cast<const i32x4*>(s_codes) + 4 * (p < npieces ? p : 0);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const i32x4 a = lp[v];
        xa[q][4 * v + 0] = a.x; xa[q][4 * v + 1] = a.y; xa[q][4 * v + 2] = a.z; xa[q][4 * v + 3] = a.w;
      }
      if (p >= npieces) {
#pragma unroll
        for (int d = 0; d < 16; ++d) xa[q][d] = 0;
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int p = lane + kWave * q;
      const i32x4* src = reinterpret_cast<const i32x4*>(da.Xq + 64 * (p < npieces ? p : 0));
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const i32x4 a = src[v];
        xa[q][4 * v + 0] = a.x; xa[q][4 * v + 1] = a.y; xa[q][4 * v + 2] = a.z; xa[q][4 * v + 3] = a.w;
      }
    }
    sx = da.xsum[0];
    sc = da.xs[0];
    // Keep the epilogue's scalar inputs here, under the weight stream's
    // latency, instead of letting them sink behind the reduction into the
    // store branch as a chain of dependent scalar loads.
    asm volatile("" ::"s"(gamma), "s"(sx), "s"(sc), "s"(yout));
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      if (lane + kWave * q >= npieces) {
#pragma unroll
        for (int d = 0; d < 16; ++d) xa[q][d] = 0;
      }
    }
  }

  int32_t mine = 0;   // lane r keeps row r's sum
  if constexpr (FUSE == kDotFuseBlock && Q > kDotHeldQ) {
    // Long rows: each piece's codes are read from LDS when its turn comes
    // (piece outer, rows inner), so only one piece of activations is held.
    int32_t accr[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int f = 0; f < 4; ++f) accr[r][f] = 0;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int p = lane + kWave * q;
      const i32x4* lp = reinterpret_cast<const i32x4*>(s_codes) + 4 * (p < npieces ? p : 0);
      int32_t xq[16];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const i32x4 a = lp[v];
        xq[4 * v + 0] = a.x; xq[4 * v + 1] = a.y; xq[4 * v + 2] = a.z; xq[4 * v + 3] = a.w;
      }
      if (p >= npieces) {
#pragma unroll
        for (int d = 0; d < 16; ++d) xq[d] = 0;
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t w4[4] = {wq[r][q].x, wq[r][q].y, wq[r][q].z, wq[r][q].w};
#pragma unroll
        for (int t = 0; t < 4; ++t) dot_word_fields(w4[t], &xq[4 * t], accr[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int32_t acc = wave_sum_i32(fields_total(accr[r]));
      if (lane == r) mine = acc;
    }
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      int32_t fa[4] = {0, 0, 0, 0};
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const uint32_t w4[4] = {wq[r][q].x, wq[r][q].y, wq[r][q].z, wq[r][q].w};
#pragma unroll
        for (int t = 0; t < 4; ++t) dot_word_fields(w4[t], &xa[q][4 * t], fa);
      }
      const int32_t acc = wave_sum_i32(fields_total(fa));
      if (lane == r) mine = acc;
    }
  }
  if (lane < R && n0 + lane < N) store_out<OUT>(yout, n0 + lane, mine - sx, gamma, sc);
}

template <int OUT, int R, int Q, int FUSE = kDotFuseNone, int WV = kDotWaves, bool NORM = false>
hipError_t launch_decode_dot_t(DecodeArgs da, hipStream_t stream) {
  const int waves = set_units(da, R);
  const int grid = (waves + WV - 1) / WV;
  k_decode_dot<OUT, R, Q, FUSE, WV, NORM><<<dim3(grid), dim3(WV * kWave), 0, stream>>>(da);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// GEMM: M > 16 tokens.
//
// A workgroup of 4 waves (WM x WN) computes a BM x BN output tile (tokens x
// weight rows).  K advances in steps of 128 through a ring of three LDS
// stages filled by direct global->LDS loads (each lane's 16 bytes land at
// base + 16 x lane), issued two steps ahead of the matrix instructions; one
// barrier per step.  The stages are three separate LDS arrays and the loop is
// unrolled by three, so every access names its stage at compile time.
//
// Stage layouts (both read conflict-free with 16-byte reads whether the LDS
// serves 8 or 16 lanes of such a read per cycle):
//   activations  BM rows of 128 bytes; piece p (k = 16p .. 16p + 15 of the
//                step) of row r sits at r * 128 + 16 * (p ^ aswz(r)),
//                aswz(r) = (r & 7) ^ ((r >> 3) & 1);
//   codes        two halves of BN 16-byte chunks; chunk (n, h) = packed words
//                4h .. 4h + 3 of code row n (k = 64h .. 64h + 63 of the step)
//                sits at h * BN * 16 + n * 16.
//
// The 32x32x32 matrix instruction takes 16 k per lane, k group lane / 32.
// Slice ks (0..3) of a step gives lane group g the k of piece 4g + ks, so a
// lane reads its column's codes for the whole step as one 16-byte chunk
// (words 4g .. 4g + 3) and the activation fragment of piece 4g + ks.  Each
// packed word is expanded once and reused across the wave's row blocks.
// Activations are the instruction's first operand and codes its second.
// The matrix cores' power draw depends on which operand holds which values:
// a loop of these instructions alone on the projection's values runs about
// 14 % faster with the low-entropy codes second than with them first, and
// since the GEMM runs at the chip's power limit, the kernel gains about as
// much.  A lane's results are then one weight row (its column of the block)
// for 16 tokens.  Its accumulators start at minus their tokens' sums of X~
// (so the code offset comes off inside the matrix sums), and the epilogue
// takes each token's scale from a table in LDS filled before the K loop.
//
// Full steps read activations at row-clamped addresses (rows past M only feed
// outputs that are not stored).  A K tail (K % 128 != 0) is one more step
// loaded through registers with exact zero fill.  Tiles are dealt so that the
// workgroups of one XCD (workgroups go round-robin over the 8 XCDs) take a
// contiguous run of tiles, sharing activation rows in that XCD's L2.
// ---------------------------------------------------------------------------
constexpr int kGemmThreads = 256;
constexpr int kGBK = 128;

struct GemmArgs {
  const uint8_t* Wp;
  const float* gamma;
  int N, K, M;
  const int8_t* Xq;
  const float* xs;
  const int32_t* xsum;
  void* Y;
  int tiles_m, tiles_n;
  int vec_out;   // 2: bf16 rows staged through LDS, 16-byte stores (k_gemm); 1: four
                 // outputs per store (split-K reduction); 0: one output per store
  int band;      // tile-order band width in column tiles (see k_gemm)
  int splits;    // K splits per tile; > 1: raw int32 partial tiles into `part`
  int32_t* part; // [splits][M][N] partial accumulators (splits > 1)
};

__device__ __forceinline__ int aswz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int a_off(int row, int piece) { return row * 128 + 16 * (piece ^ aswz(row)); }
template <int BN>
__device__ __forceinline__ int b_off(int row, int word) {
  return (word >> 2) * BN * 16 + row * 16 + 4 * (word & 3);
}

// vmcnt(n) only (expcnt and lgkmcnt left at their maxima).
template <int NV>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(NV >= 0 && NV < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((NV & 0xF) | ((NV >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup rendezvous without a memory fence.  __syncthreads() would also
// wait for every direct-to-LDS load still in flight (its release fence covers
// them), draining the prefetch ring; here each wave first waits only for the
// loads of the stage about to be read (wait_vmcnt), whose LDS writes are done
// when the counter drops.  The empty asm statements keep the compiler from
// moving memory accesses across the barrier.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait until this wave's LDS reads are done (lgkmcnt 0; other counters free).
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));
}

// One stage's fragments in registers: the lane's code words and its
// activation rows for the four 32-wide k sub-steps.
template <int MB, int NB>
struct GemmFrag {
  i32x4 bw[NB];
  i32x4 af[kGBK / 32][MB];
};

template <int BN, int MB, int NB>
__device__ __forceinline__ void gemm_read(const int8_t* __restrict__ Ac,
                                          const uint8_t* __restrict__ Bc, int a_row0, int b_row0,
                                          int lane_sw, int g2, GemmFrag<MB, NB>& f) {
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    f.bw[nb] = *reinterpret_cast<const i32x4*>(Bc + g2 * BN * 16 + (b_row0 + nb * 32) * 16);
#pragma unroll
  for (int ks = 0; ks < kGBK / 32; ++ks)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      f.af[ks][mb] = *reinterpret_cast<const i32x4*>(Ac + (a_row0 + mb * 32) * 128 +
                                                     16 * ((4 * g2 + ks) ^ lane_sw));
}

template <int MB, int NB, int NA>
__device__ __forceinline__ void gemm_mma(const GemmFrag<MB, NB>& f, i32x16 (&acc)[NA][MB][NB]);

// One step with fragments read one stage ahead: issue the direct loads of a
// later stage into (An, Bn), read the next stage's fragments from (Ar, Br)
// into nxt, and run the matrix instructions on cur.  As in gemm_step, the
// __restrict__ qualifiers let the compiler see that the stage being read is
// not the one being filled, so it waits for no load in flight.
template <int BN, int MB, int NB, int A_INS, int B_INS, int NA>
__device__ __forceinline__ void gemm_step_pf(const int8_t* __restrict__ Ar,
                                             const uint8_t* __restrict__ Br,
                                             int8_t* __restrict__ An, uint8_t* __restrict__ Bn,
                                             const int8_t* const (&asrc)[A_INS],
                                             const uint8_t* const (&bsrc)[B_INS],
                                             const int (&bblk)[B_INS], int k0n, int wave,
                                             int a_row0, int b_row0, int lane_sw, int g2,
                                             const GemmFrag<MB, NB>& cur, GemmFrag<MB, NB>& nxt,
                                             i32x16 (&acc)[NA][MB][NB]) {
#pragma unroll
  for (int qi = 0; qi < A_INS; ++qi)
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(asrc[qi] + k0n),
                                     static_cast<void*>(An + (qi * 4 + wave) * 1024), 16, 0, 0);
#pragma unroll
  for (int qi = 0; qi < B_INS; ++qi)
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(bsrc[qi] + k0n / 4),
                                     static_cast<void*>(Bn + bblk[qi] * 1024), 16, 0, 0);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    nxt.bw[nb] = *reinterpret_cast<const i32x4*>(Br + g2 * BN * 16 + (b_row0 + nb * 32) * 16);
#pragma unroll
  for (int ks = 0; ks < kGBK / 32; ++ks)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      nxt.af[ks][mb] = *reinterpret_cast<const i32x4*>(Ar + (a_row0 + mb * 32) * 128 +
                                                       16 * ((4 * g2 + ks) ^ lane_sw));
  gemm_mma<MB, NB, NA>(cur, acc);
}

template <int MB, int NB, int NA>
__device__ __forceinline__ void gemm_mma(const GemmFrag<MB, NB>& f, i32x16 (&acc)[NA][MB][NB]) {
#pragma unroll
  for (int ks = 0; ks < kGBK / 32; ++ks) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const i32x4 bf = expand_codes((uint32_t)f.bw[nb][ks]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[ks % NA][mb][nb] = mfma_i8_32x32x32(f.af[ks][mb], bf, acc[ks % NA][mb][nb]);
    }
  }
}

// One pipeline step: issue the direct loads of a later stage into (An, Bn)
// and run the matrix instructions on the current stage (Ac, Bc).  The
// __restrict__ qualifiers tell the compiler the two stages are disjoint, so it
// need not wait for the loads in flight before reading the current stage, and
// it schedules the fragment reads itself.
template <int BN, int MB, int NB, int A_INS, int B_INS, int NA>
__device__ __forceinline__ void gemm_step(const int8_t* __restrict__ Ac, const uint8_t* __restrict__ Bc,
                                          int8_t* __restrict__ An, uint8_t* __restrict__ Bn,
                                          bool do_issue, const int8_t* const (&asrc)[A_INS],
                                          const uint8_t* const (&bsrc)[B_INS],
                                          const int (&bblk)[B_INS], int k0n, int wave,
                                          int a_row0, int b_row0, int lane_sw, int g2,
                                          i32x16 (&acc)[NA][MB][NB]) {
  if (do_issue) {
#pragma unroll
    for (int qi = 0; qi < A_INS; ++qi)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(asrc[qi] + k0n),
                                       static_cast<void*>(An + (qi * 4 + wave) * 1024), 16, 0, 0);
#pragma unroll
    for (int qi = 0; qi < B_INS; ++qi)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(bsrc[qi] + k0n / 4),
                                       static_cast<void*>(Bn + bblk[qi] * 1024), 16, 0, 0);
  }
  constexpr int KS = kGBK / 32;
  i32x4 bw[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    bw[nb] = *reinterpret_cast<const i32x4*>(Bc + g2 * BN * 16 + (b_row0 + nb * 32) * 16);
  i32x4 af[KS][MB];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      af[ks][mb] = *reinterpret_cast<const i32x4*>(Ac + (a_row0 + mb * 32) * 128 +
                                                    16 * ((4 * g2 + ks) ^ lane_sw));
  // Sub-step ks accumulates into set ks % NA: with few blocks per wave the
  // matrix instructions of a step would otherwise form one dependent chain.
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const i32x4 bf = expand_codes((uint32_t)bw[nb][ks]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[ks % NA][mb][nb] = mfma_i8_32x32x32(af[ks][mb], bf, acc[ks % NA][mb][nb]);
    }
  }
}

// WPE: minimum waves per SIMD the registers must allow (1: the compiler's
// own choice).  128 x 256 tiles need 2 (their 128 accumulator registers
// would otherwise push the compiler to one wave per SIMD).
template <bool kAligned64, int OUT, int BM, int BN, int WM, int WN, int NS, bool PF, int WPE>
__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(WPE)))
void k_gemm(GemmArgs ga) {
  static_assert(WM * WN == kGemmThreads / kWave, "4 waves");
  static_assert(NS >= 2 && NS <= 8, "ring depth");
  constexpr int MB = BM / WM / 32, NB = BN / WN / 32;   // 32x32 blocks per wave
  static_assert(MB >= 1 && NB >= 1 && BN % 64 == 0, "tile");
  // Independent accumulator sets (added exactly at the end): at least four
  // independent matrix-instruction chains per wave.
  constexpr int NA = MB * NB >= 4 ? 1 : 4 / (MB * NB);
  constexpr int A_INS = BM / 8 / 4;            // 1 KB direct loads per wave per stage (8 rows each)
  constexpr int B_BLK = BN / 32;               // 1 KB blocks of codes per stage (64 chunks each)
  constexpr int B_INS = (B_BLK + 3) / 4;       // per wave
  static_assert(A_INS >= 1, "tile");
  // One array per stage, so every access names its stage at compile time.
  // (sA2 also stages wave 2's epilogue rows, so it keeps 4 KB at NS = 2.)
#define BL_SA(i) sA##i[NS > i ? BM * 128 : (i == 2 ? 4096 : 16)]
#define BL_SB(i) sB##i[NS > i ? BN * 32 : 16]
  __shared__ __attribute__((aligned(1024))) int8_t BL_SA(0), BL_SA(1), BL_SA(2), BL_SA(3),
      BL_SA(4), BL_SA(5), BL_SA(6), BL_SA(7);
  __shared__ __attribute__((aligned(1024))) uint8_t BL_SB(0), BL_SB(1), BL_SB(2), BL_SB(3),
      BL_SB(4), BL_SB(5), BL_SB(6), BL_SB(7);
#undef BL_SA
#undef BL_SB
  __shared__ __attribute__((aligned(16))) float tok_scale[BM];
  int8_t* const sA[8] = {sA0, sA1, sA2, sA3, sA4, sA5, sA6, sA7};
  uint8_t* const sB[8] = {sB0, sB1, sB2, sB3, sB4, sB5, sB6, sB7};

  // Every argument the prologue uses, requested in one round of scalar loads
  // (left to itself the compiler loads them where first used, in three
  // dependent rounds, each waiting for the last).
  asm volatile("" ::"s"(ga.Wp), "s"(ga.Xq), "s"(ga.xsum), "s"(ga.xs), "s"(ga.N), "s"(ga.K),
               "s"(ga.M), "s"(ga.tiles_m), "s"(ga.tiles_n), "s"(ga.band), "s"(ga.splits));
  __builtin_amdgcn_sched_barrier(0);
  const int N = ga.N, K = ga.K, M = ga.M;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int r32 = lane & 31, g2 = lane >> 5;   // row/column within a 32 block, k group
  const int kw = K / 16;

  // Bijective XCD-aware tile order.  XCD x (= b % 8) takes positions
  // [x q + min(x, r), ...) of the tile order, T = 8 q + r.  The order walks
  // bands of `band` column tiles; inside a band, token row tiles, then the
  // band's columns.  The workgroups resident on one XCD then share a few
  // activation row blocks and one band of code blocks in that XCD's L2.
  // With K split S ways, the order runs over (tile, split) items, the S
  // splits of a tile adjacent.
  const int S = ga.splits;
  const int TT = ga.tiles_m * ga.tiles_n * S;
  const int b = blockIdx.x;
  const int xcd = b & 7, q8 = TT >> 3, r8 = TT & 7;
  const int item = xcd * q8 + min(xcd, r8) + (b >> 3);
  const int t = item / S, split = item - t * S;
  const int band_tiles = ga.tiles_m * ga.band;
  const int bi = t / band_tiles;
  const int within = t - bi * band_tiles;
  const int bw = min(ga.band, ga.tiles_n - bi * ga.band);
  const int tm = within / bw, tn = bi * ga.band + within % bw;
  const int m0 = tm * BM, n0 = tn * BN;
  // This item's full K steps [kb, kb + nkf); the K tail goes to the last split.
  const int nk_all = K / kGBK;
  const int per_split = (nk_all + S - 1) / S;
  const int kb = min(split * per_split, nk_all);
  const bool has_tail = (K % kGBK) != 0 && split == S - 1;

  // Per-lane source addresses of the direct loads (k offset added per step).
  // Activation block blk holds rows 8 blk .. 8 blk + 7; lane l fills slot
  // l & 7 of row 8 blk + (l >> 3), i.e. piece (l & 7) ^ aswz(row).
  const int8_t* asrc[A_INS];
#pragma unroll
  for (int qi = 0; qi < A_INS; ++qi) {
    const int blk = qi * 4 + wave;
    const int r = blk * 8 + (lane >> 3);
    const int piece = (lane & 7) ^ aswz(r);
    asrc[qi] = ga.Xq + (int64_t)min(m0 + r, M - 1) * K + (int64_t)kb * kGBK + 16 * piece;
  }
  // Code block bb holds half h = bb / (BN / 64) of rows 64 (bb % (BN / 64))
  // + lane.  Every wave issues B_INS code loads per stage, so all waves have
  // the same count in flight; a wave past the last block repeats it (same
  // bytes to the same place).
  const uint8_t* bsrc[B_INS];
  int bblk[B_INS];
#pragma unroll
  for (int qi = 0; qi < B_INS; ++qi) {
    bblk[qi] = min(qi * 4 + wave, B_BLK - 1);
    const int h = bblk[qi] / (BN / 64);
    const int r = (bblk[qi] % (BN / 64)) * 64 + lane;
    bsrc[qi] = ga.Wp + (int64_t)min(n0 + r, N - 1) * (K / 4) + (int64_t)kb * (kGBK / 4) + 16 * h;
  }
  auto issue = [&](int kt, int8_t* A, uint8_t* B) {
    const int k0 = kt * kGBK;
#pragma unroll
    for (int qi = 0; qi < A_INS; ++qi)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(asrc[qi] + k0),
                                       static_cast<void*>(A + (qi * 4 + wave) * 1024), 16, 0, 0);
#pragma unroll
    for (int qi = 0; qi < B_INS; ++qi)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(bsrc[qi] + k0 / 4),
                                       static_cast<void*>(B + bblk[qi] * 1024), 16, 0, 0);
  };

  i32x16 acc_sets[NA][MB][NB];
#pragma unroll
  for (int h = 0; h < NA; ++h)
#pragma unroll
    for (int a = 0; a < MB; ++a)
#pragma unroll
      for (int c = 0; c < NB; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc_sets[h][a][c][e] = 0;
  // Without a K split, each accumulator of the first set starts at minus its
  // token's sum of X~: the matrix sums then end at sum_k (c - 1) x~ = the
  // exact W~ X~ product, with no subtraction per output in the epilogue.
  // (Register 4 i + j of block (mb, nb) belongs to token row
  // mb * 32 + 8 i + 4 g2 + j of the wave's sub-tile; rows past M repeat row
  // M - 1, and their outputs are not stored.)
  if (S == 1) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = min(m0 + wm * MB * 32 + mb * 32 + 8 * (e >> 2) + 4 * g2 + (e & 3), M - 1);
        const int32_t sx = ga.xsum[m];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc_sets[0][mb][nb][e] = -sx;
      }
  }

  // The tile's token scales for the epilogue, loaded now so that the loads
  // are long done by then (rows past M repeat row M - 1).
  if (tid < BM) tok_scale[tid] = ga.xs[min(m0 + tid, M - 1)];

  // Fragment rows of this lane; aswz of an activation row depends only on
  // r32 (row blocks are 32 apart).
  const int a_row0 = wm * MB * 32 + r32;
  const int b_row0 = wn * NB * 32 + r32;
  const int lane_sw = aswz(r32);

  // The ring runs NS - 1 stages ahead.  Every step issues exactly NLD loads
  // (the last steps re-load the last stage into buffers nobody reads
  // again), so before step kt the only loads younger than stage kt's are
  // those of the NS - 2 stages after it, and one unconditional
  // vmcnt((NS - 2) NLD) wait suffices.  Uniform counts also let the compiler
  // see that the wait retires the stage being read, so it adds no drain of
  // its own.
  constexpr int NLD = A_INS + B_INS;
  const int nkf = min(per_split, nk_all - kb);   // full steps of this item
  if constexpr (PF) {
    // Fragments one step ahead in registers.  At step st the fragments of
    // stage st are already in registers (read during step st - 1), so the
    // matrix instructions of step st run while the LDS reads of stage
    // st + 1 are in flight; with one workgroup per CU nothing else would
    // hide that latency.  The ring is issued NS stages deep: before step st,
    // stages up to st + NS - 1 are issued, stage st's buffer is released at
    // the barrier of step st (after every wave's reads of it), and refilled
    // with stage st + NS.
    constexpr int U = NS % 2 == 0 ? NS : 2 * NS;   // stage and fragment indices static
    GemmFrag<MB, NB> fr[2];
    if (nkf > 0) {
#pragma unroll
      for (int s = 0; s < NS; ++s) issue(min(s, nkf - 1), sA[s], sB[s]);
      wait_vmcnt<(NS - 1) * NLD>();
      stage_barrier();
      gemm_read<BN, MB, NB>(sA[0], sB[0], a_row0, b_row0, lane_sw, g2, fr[0]);
    }
    for (int kt = 0; kt < nkf; kt += U) {
#pragma unroll
      for (int s = 0; s < U; ++s) {
        if (kt + s >= nkf) break;
        // This wave's reads of stage st are done and its loads of stage
        // st + 1 have landed; after the barrier the same holds for every
        // wave, so stage st + 1 is complete and stage st's buffer is free.
        wait_lgkm0();
        wait_vmcnt<(NS - 2) * NLD>();
        stage_barrier();
        gemm_step_pf<BN, MB, NB, A_INS, B_INS, NA>(
            sA[(s + 1) % NS], sB[(s + 1) % NS], sA[s % NS], sB[s % NS], asrc, bsrc, bblk,
            min(kt + s + NS, nkf - 1) * kGBK, wave, a_row0, b_row0, lane_sw, g2, fr[s & 1],
            fr[(s + 1) & 1], acc_sets);
      }
    }
  } else {
  if (nkf > 0) {
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) issue(min(s, nkf - 1), sA[s], sB[s]);
  }
  for (int kt = 0; kt < nkf; kt += NS) {
    // A break leaves the rest, so no path reaches a step without the loads
    // of the steps before it.
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (kt + s >= nkf) break;
      wait_vmcnt<(NS - 2) * NLD>();
      // Also orders this wave's reads of stage kt + s - 1 (the buffer
      // refilled below) before the other waves' refills: every wave has
      // finished that step when it reaches this barrier.
      stage_barrier();
      gemm_step<BN, MB, NB, A_INS, B_INS, NA>(sA[s], sB[s], sA[(s + NS - 1) % NS],
                                              sB[(s + NS - 1) % NS], true, asrc, bsrc, bblk,
                                              min(kt + s + NS - 1, nkf - 1) * kGBK, wave, a_row0,
                                              b_row0, lane_sw, g2, acc_sets);
    }
  }
  }
  // No direct load may still be writing LDS when the tail refills a stage or
  // the workgroup ends.
  wait_vmcnt<0>();
  if (has_tail) {
    // Tail step through registers, exact zero fill; the barrier below waits
    // until no wave reads a stage any more.
    int8_t* A = sA0;
    uint8_t* B = sB0;
    const int k0 = nk_all * kGBK;
    __syncthreads();
    for (int qd = tid; qd < BM * 8; qd += kGemmThreads) {
      const int r = qd >> 3, piece = qd & 7;
      const int m = m0 + r, k = k0 + 16 * piece;
      i32x4 v = {0, 0, 0, 0};
      if (m < M && k < K) v = *reinterpret_cast<const i32x4*>(ga.Xq + (int64_t)m * K + k);
      *reinterpret_cast<i32x4*>(A + a_off(r, piece)) = v;
    }
    for (int qd = tid; qd < BN * 8; qd += kGemmThreads) {
      const int r = qd >> 3, word = qd & 7;
      const int n = min(n0 + r, N - 1);
      const uint32_t* row = reinterpret_cast<const uint32_t*>(ga.Wp + (int64_t)n * (K / 4));
      *reinterpret_cast<uint32_t*>(B + b_off<BN>(r, word)) = load_word(row, k0 / 16 + word, kw);
    }
    __syncthreads();
    gemm_step<BN, MB, NB, A_INS, B_INS, NA>(A, B, nullptr, nullptr, false, asrc, bsrc, bblk, 0,
                                            wave, a_row0, b_row0, lane_sw, g2, acc_sets);
  }
  i32x16 (&acc)[MB][NB] = acc_sets[0];
#pragma unroll
  for (int h = 1; h < NA; ++h)
#pragma unroll
    for (int a = 0; a < MB; ++a)
#pragma unroll
      for (int c = 0; c < NB; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[a][c][e] += acc_sets[h][a][c][e];

  // Epilogue: lane (r32, g2), register 4 i + j of block (mb, nb) holds the
  // output of token m0 + (row block) + 8 i + 4 g2 + j and weight row
  // n0 + (column block) + r32.  For a fixed register the 32 lanes of a half
  // hold 32 consecutive weight rows of one token: consecutive addresses.
  if (S > 1) {
    // Raw partial accumulators of this split; the reduction kernel adds the
    // splits, subtracts the code offset and rescales.
    int32_t* P = ga.part + (int64_t)split * M * N;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int n = n0 + wn * NB * 32 + nb * 32 + r32;
        if (n >= N) continue;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = m0 + wm * MB * 32 + mb * 32 + 8 * (e >> 2) + 4 * g2 + (e & 3);
          if (m < M) P[(int64_t)m * N + n] = acc[mb][nb][e];
        }
      }
    }
    return;
  }
  const float gamma = ga.gamma[0];
  // The token scales are in LDS, and (for the staged stores) every wave is
  // done with the stage buffers.
  __syncthreads();
  if constexpr (OUT == kOutBF16) {
    if (ga.vec_out == 2) {
      // Rows of 16-byte pieces through LDS: each wave stages one 32-token
      // block of its sub-tile at a time in a stage buffer of its own (4 KB or
      // 2 KB), then writes whole row segments (NB * 64 bytes) with 16-byte
      // stores.  Piece c of staged row r sits at slot c ^ ((r / RPL) % CH),
      // which keeps the 16-byte reads conflict-free.
      constexpr int CH = NB * 4;            // 16-byte pieces per staged row
      constexpr int RPL = 16 / CH;          // staged rows per 256-byte bank row
      static_assert(32 * CH * 16 <= BN * 32, "a code stage holds one block");
      uint8_t* buf = wave == 0 ? reinterpret_cast<uint8_t*>(sA0)
                   : wave == 1 ? reinterpret_cast<uint8_t*>(sA1)
                   : wave == 2 ? reinterpret_cast<uint8_t*>(sA2) : sB0;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int t0 = wm * MB * 32 + mb * 32;   // the block's first token in the tile
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r0 = 8 * i + 4 * g2;          // staged rows r0 .. r0 + 3
          const float4 sc = *reinterpret_cast<const float4*>(tok_scale + t0 + r0);
          const float scj[4] = {sc.x, sc.y, sc.z, sc.w};
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const int col = nb * 32 + r32;        // bf16 column of the staged row
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int r = r0 + j;
              const float y = ((float)acc[mb][nb][4 * i + j] * gamma) * scj[j];
              // The hardware conversion (v_cvt_pk_bf16_f32) rounds to
              // nearest even: the same bits as f32_to_bf16_rne for every
              // non-NaN value, in one instruction.
              *reinterpret_cast<__bf16*>(buf + r * (CH * 16) + 16 * ((col >> 3) ^ ((r / RPL) % CH)) +
                                         2 * (col & 7)) = (__bf16)y;
            }
          }
        }
        // The wave's LDS accesses complete in order, so its reads below see
        // its writes above, and the next block's writes follow these reads.
#pragma unroll
        for (int q = 0; q < 32 * CH / kWave; ++q) {
          const int row = q * (kWave / CH) + lane / CH;
          const int c = lane % CH;
          const uint4 v = *reinterpret_cast<const uint4*>(
              buf + row * (CH * 16) + 16 * (c ^ ((row / RPL) % CH)));
          const int m = m0 + t0 + row;
          const int n = n0 + wn * NB * 32 + 8 * c;
          if (m < M && n < N)
            *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(ga.Y) + (int64_t)m * N + n) = v;
        }
      }
      return;
    }
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int t0 = wm * MB * 32 + mb * 32;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r0 = 8 * i + 4 * g2;
      const float4 sc = *reinterpret_cast<const float4*>(tok_scale + t0 + r0);
      const float scj[4] = {sc.x, sc.y, sc.z, sc.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = m0 + t0 + r0 + j;
        if (m >= M) continue;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int n = n0 + wn * NB * 32 + nb * 32 + r32;
          if (n < N)
            store_out<OUT>(ga.Y, (int64_t)m * N + n, acc[mb][nb][4 * i + j], gamma, scj[j]);
        }
      }
    }
  }
}

constexpr int kMaxSplits = 4;   // K splits of one projection (gemm_cfg's maximum)

// Sum of the K splits of every output, then the epilogue: thread i handles
// outputs 4i .. 4i + 3 of the flattened [M][N] tile set when N % 4 == 0 (one
// vector load per split), else one output.
template <int OUT>
__global__ __launch_bounds__(256) void k_splitk_reduce(GemmArgs ga) {
  const int M = ga.M, N = ga.N, S = ga.splits;
  const int64_t MN = (int64_t)M * N;
  const float gamma = ga.gamma[0];
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (N % 4 == 0) {
    const int64_t e = 4 * i;
    if (e >= MN) return;
    const int m = (int)(e / N);
    // Every split's partials are requested before any is added (S <= 4),
    // so the loads overlap instead of following one another.
    i32x4 w[kMaxSplits];
#pragma unroll
    for (int sp = 0; sp < kMaxSplits; ++sp)
      w[sp] = sp < S ? *reinterpret_cast<const i32x4*>(ga.part + sp * MN + e) : i32x4{0, 0, 0, 0};
    i32x4 v = w[0];
#pragma unroll
    for (int sp = 1; sp < kMaxSplits; ++sp) {
      v.x += w[sp].x; v.y += w[sp].y; v.z += w[sp].z; v.w += w[sp].w;
    }
    const int32_t sx = ga.xsum[m];
    v.x -= sx; v.y -= sx; v.z -= sx; v.w -= sx;
    if (ga.vec_out) {
      store_out4<OUT>(ga.Y, e, v, gamma, ga.xs[m]);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) store_out<OUT>(ga.Y, e + j, v[j], gamma, ga.xs[m]);
    }
  } else {
    if (i >= MN) return;
    const int m = (int)(i / N);
    int32_t w[kMaxSplits];
#pragma unroll
    for (int sp = 0; sp < kMaxSplits; ++sp) w[sp] = sp < S ? ga.part[sp * MN + i] : 0;
    int32_t a = 0;
#pragma unroll
    for (int sp = 0; sp < kMaxSplits; ++sp) a += w[sp];
    store_out<OUT>(ga.Y, i, a - ga.xsum[m], gamma, ga.xs[m]);
  }
}

// ---------------------------------------------------------------------------
// Skinny projections: 2 to 64 tokens (M <= 16 TG), K % 64 == 0.
//
// Between the single-token decode and the GEMM.  A workgroup owns RB blocks
// of 16 weight rows and runs NWK waves per block; K advances in chunks of
// CK = 256 NWK, and wave kw of a block takes chunk group kw (256 k) of every
// chunk.  Per chunk group a lane takes one 16-byte piece of its row (64
// codes) and issues 4 TG matrix instructions (16x16x64), one per token group.
// Activations and codes both stream through an LDS ring of NS = SP + 1
// stages, SP chunks ahead, filled with direct loads of the same count per
// wave and step, so one vmcnt wait per step retires exactly the stage about
// to be read (a ring of registers carried across the loop would make the
// compiler drain every load at the loop head).  With about one workgroup per
// CU (about 256 workgroups of RB NWK = 8 waves, or RB = 1 with 4 waves on
// narrow outputs), the activations are read from L2 about once per CU rather
// than once per output tile.
//
// Stage layouts (16-byte pieces XOR-swizzled by row, so that the lanes of a
// fragment read, 16 rows and one piece, fall in different bank groups):
//   activations [16 TG token rows][CK bytes], piece q of row r at q ^ (r & 15);
//   codes       [RB][16 rows][64 NWK bytes], piece q of row r at q ^ (r & (4 NWK - 1)).
// Rows past M or N and pieces past K are loaded from clamped addresses
// (garbage): past M or N the outputs are not stored; past K the codes are
// masked to 0, which contributes nothing.
// ---------------------------------------------------------------------------
// One step of k_skinny: issue the direct loads of a later chunk into (An, Bn)
// and run the current chunk from (Ac, Bc).  The __restrict__ qualifiers tell
// the compiler the two stages are disjoint (as in gemm_step).
template <int TG, int NWK, typename Issue>
__device__ __forceinline__ void skinny_step(const int8_t* __restrict__ Ac,
                                            const uint8_t* __restrict__ Bc,
                                            int8_t* __restrict__ An, uint8_t* __restrict__ Bn,
                                            Issue issue, int wr, int qw, int j, uint32_t wmask,
                                            i32x4 (&acc)[TG]) {
  constexpr int CK = 256 * NWK, WROW = 64 * NWK, WSW = 4 * NWK - 1;
  issue(An, Bn);
  const uint4 wv = *reinterpret_cast<const uint4*>(Bc + wr * WROW + 16 * (qw ^ (wr & WSW)));
  const uint32_t w4[4] = {wv.x & wmask, wv.y & wmask, wv.z & wmask, wv.w & wmask};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const i32x4 b = expand_codes(w4[t]);
    const int q = 4 * qw + t;                   // 16-byte piece of the chunk (k = 16 q ..)
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
      const int r = 16 * tg + j;
      const i32x4 a = *reinterpret_cast<const i32x4*>(Ac + r * CK + 16 * (q ^ (r & 15)));
      acc[tg] = mfma_i8_16x16x64(a, b, acc[tg]);
    }
  }
}

// Work unit: one workgroup (RB row blocks of one projection).
// TS: the tokens split in halves of 16 TG, one workgroup per (row group,
// half); the halves of a row group sit 8 workgroups apart, on one XCD, when
// the row groups are a multiple of 8.
template <int TG, int RB, int NWK, int SP, int OUT, bool TS = false>
__global__ __launch_bounds__(RB * NWK * kWave) void k_skinny(DecodeArgs da) {
  constexpr int NWV = RB * NWK;               // waves
  constexpr int CK = 256 * NWK;               // k per chunk
  constexpr int NS = SP + 1;                  // ring stages
  constexpr int ROWS = 16 * TG;
  constexpr int XSTAGE = ROWS * CK;           // activation bytes per stage
  constexpr int XBLOCKS = XSTAGE / 1024;      // 1 KB direct loads per stage
  constexpr int XL = (XBLOCKS + NWV - 1) / NWV;   // per wave (the last one repeated)
  constexpr int WROW = 64 * NWK;              // code bytes of one row per chunk
  constexpr int WSTAGE = RB * 16 * WROW;      // = NWV KB: one direct load per wave
  constexpr int NLD = XL + 1;                 // loads per wave per step
  constexpr int WSW = 4 * NWK - 1;            // code piece swizzle mask
  static_assert(XSTAGE % 1024 == 0 && WSTAGE == NWV * 1024, "stage");
  static_assert(NS >= 2 && NS <= 4, "ring depth");
  static_assert(RB * (NWK - 1) * TG * kWave * 16 <= XSTAGE, "partial tiles fit stage 0");
  // One array per stage, so that every access names its stage at compile
  // time and the compiler can tell the stage being read from the one being
  // filled (one array of stages would make it wait for every load in flight).
#define BL_SX(i) sX##i[NS > i ? XSTAGE : 16]
#define BL_SW(i) sW##i[NS > i ? WSTAGE : 16]
  __shared__ __attribute__((aligned(1024))) int8_t BL_SX(0), BL_SX(1), BL_SX(2), BL_SX(3);
  __shared__ __attribute__((aligned(1024))) uint8_t BL_SW(0), BL_SW(1), BL_SW(2), BL_SW(3);
#undef BL_SX
#undef BL_SW
  int8_t* const sX[4] = {sX0, sX1, sX2, sX3};
  uint8_t* const sW[4] = {sW0, sW1, sW2, sW3};

  // With K split S ways (one projection), the S workgroups of a row group
  // are adjacent and split sp takes chunks [cb, cb + nch).
  const int S = da.splits > 1 ? da.splits : 1;
  int wg = blockIdx.x / S, half = 0;
  if constexpr (TS) {
    const int units = (int)(gridDim.x >> 1);
    if ((units & 7) == 0) {
      const int slot = (int)blockIdx.x >> 3;
      wg = (slot >> 1) * 8 + ((int)blockIdx.x & 7);
      half = slot & 1;
    } else {
      wg = (int)blockIdx.x % units;
      half = (int)blockIdx.x / units;
    }
  }
  const int sp = TS ? 0 : (int)blockIdx.x - wg * S;
  const DecodeView view = decode_view(da, wg);
  // this workgroup's tokens: [mh, mh + M)
  const int mh = half * 16 * TG;
  const int N = view.N, K = da.K, M = TS ? min(da.M - mh, 16 * TG) : da.M;
  const int8_t* const Xq = da.Xq + (int64_t)mh * K;
  const float* const xsc = da.xs + mh;
  const int32_t* const xsm = da.xsum + mh;
  const uint8_t* const Wp = view.Wp;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rb = wave / NWK, kw = wave - rb * NWK;
  const int j = lane & 15, g = lane >> 4;
  const int nb0 = view.unit * RB;             // first row block of the workgroup
  const int npieces = K / 64;
  const int kbytes = K / 4;
  const int nch_all = (K + CK - 1) / CK;
  const int cps = (nch_all + S - 1) / S;
  const int cb = min(sp * cps, nch_all);
  const int nch = min(cps, nch_all - cb);     // >= 1 (skinny_splits sizes S so)

  // Epilogue inputs now, so no memory round trip follows the reduction.
  const float gamma = view.gamma[0];
  int32_t sxv[TG][4];
  float scv[TG][4];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = min(16 * tg + 4 * g + r, M - 1);
      sxv[tg][r] = xsm[m];
      scv[tg][r] = xsc[m];
    }

  // Direct loads of chunk c: activation blocks wave, wave + NWV, ... and the
  // code block `wave`.  Lane l fills the 16-byte slot at 1024 b + 16 l of its
  // block: activation row r = slot / CK, position q' within the row, source
  // piece q' ^ (r & 15); code row block b / NWK, row r = slot / WROW within
  // the workgroup's stage, position q', source piece q' ^ (r & WSW).
  auto issue = [&](int c, int8_t* A, uint8_t* B) {
#pragma unroll
    for (int i = 0; i < XL; ++i) {
      const int b = min(wave + NWV * i, XBLOCKS - 1);
      const int off = 1024 * b + 16 * lane;
      const int r = off / CK;
      const int q = ((off % CK) / 16) ^ (r & 15);
      const int m = min(r, M - 1);
      const int k = min((cb + c) * CK + 16 * q, K - 16);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(Xq + (int64_t)m * K + k),
                                       static_cast<void*>(A + 1024 * b), 16, 0, 0);
    }
    {
      const int off = 1024 * wave + 16 * lane;
      const int r = off / WROW;                 // row within the workgroup's 16 RB rows
      const int q = ((off % WROW) / 16) ^ (r & WSW);
      const int n = min(16 * nb0 + r, N - 1);
      const int kb = min((cb + c) * (CK / 4) + 16 * q, kbytes - 16);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(Wp + (int64_t)n * kbytes + kb),
                                       static_cast<void*>(B + 1024 * wave), 16, 0, kLdsLoadOnce);
    }
  };

  i32x4 acc[TG];
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) acc[tg] = i32x4{0, 0, 0, 0};

  const int wr = 16 * rb + j;                   // this lane's code row in the stage
  const int qw = 4 * kw + g;                    // and its piece of the chunk
#pragma unroll
  for (int s = 0; s < SP; ++s) issue(min(s, nch - 1), sX[s], sW[s]);
  for (int c0 = 0; c0 < nch; c0 += NS) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int c = c0 + s;
      if (c >= nch) break;
      // This wave's loads of chunk c have landed (the SP - 1 younger chunks
      // may still be in flight); after the barrier every wave's have, and
      // every wave has finished chunk c - 1, whose stage is refilled below.
      wait_vmcnt<(SP - 1) * NLD>();
      stage_barrier();
      // pieces past K: code 0 (the mask does not depend on the loaded value)
      const uint32_t wmask = (cb + c) * (CK / 64) + qw < npieces ? 0xffffffffu : 0u;
      skinny_step<TG, NWK>(sX[s], sW[s], sX[(s + SP) % NS], sW[(s + SP) % NS],
                           [&](int8_t* An, uint8_t* Bn) { issue(min(c + SP, nch - 1), An, Bn); },
                           wr, qw, j, wmask, acc);
    }
  }
  wait_vmcnt<0>();

  // Waves kw > 0 hand their partial tiles to wave kw = 0 of their row block.
  if constexpr (NWK > 1) {
    __syncthreads();   // every wave is done with the stages
    i32x4* red = reinterpret_cast<i32x4*>(sX0);   // [RB][NWK - 1][TG][64]
    if (kw > 0) {
#pragma unroll
      for (int tg = 0; tg < TG; ++tg)
        red[((rb * (NWK - 1) + kw - 1) * TG + tg) * kWave + lane] = acc[tg];
    }
    __syncthreads();
    if (kw > 0) return;
#pragma unroll
    for (int w2 = 0; w2 < NWK - 1; ++w2)
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) {
        const i32x4 o = red[((rb * (NWK - 1) + w2) * TG + tg) * kWave + lane];
        acc[tg].x += o.x; acc[tg].y += o.y; acc[tg].z += o.z; acc[tg].w += o.w;
      }
  }
  // Lane (j, g) register r of token group tg: token 16 tg + 4 g + r, row n.
  const int n = 16 * (nb0 + rb) + j;
  if (n >= N) return;
  if (S > 1) {
    // Raw partial sums of this split; k_splitk_reduce adds the splits and
    // applies the epilogue.
    int32_t* P = da.part + (int64_t)sp * M * N;
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
      const int32_t v[4] = {acc[tg].x, acc[tg].y, acc[tg].z, acc[tg].w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 16 * tg + 4 * g + r;
        if (m < M) P[(int64_t)m * N + n] = v[r];
      }
    }
    return;
  }
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
    const int32_t v[4] = {acc[tg].x, acc[tg].y, acc[tg].z, acc[tg].w};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 16 * tg + 4 * g + r;
      if (m < M)
        store_out<OUT>(view.Y, (int64_t)(mh + m) * N + n, v[r] - sxv[tg][r], gamma, scv[tg][r]);
    }
  }
}

// The tokens as two halves of 16 TG (TS form of k_skinny; no K split)
template <int TG, int RB, int NWK, int SP, int OUT>
hipError_t launch_skinny_ts_t(DecodeArgs da, hipStream_t stream) {
  const int grid = set_units(da, 16 * RB) * 2;
  k_skinny<TG, RB, NWK, SP, OUT, true><<<dim3(grid), dim3(RB * NWK * kWave), 0, stream>>>(da);
  return hipGetLastError();
}

template <int TG, int RB, int NWK, int SP, int OUT>
hipError_t launch_skinny_t(DecodeArgs da, hipStream_t stream) {
  const int grid = set_units(da, 16 * RB) * (da.splits > 1 ? da.splits : 1);
  k_skinny<TG, RB, NWK, SP, OUT><<<dim3(grid), dim3(RB * NWK * kWave), 0, stream>>>(da);
  return hipGetLastError();
}

// K split S ways over one projection: raw partial sums into `part`
// ([S][M][N] int32, exact), then k_splitk_reduce adds them in split order
// and applies the epilogue.
template <int TG, int RB, int NWK, int SP, int OUT>
hipError_t launch_skinny_split_t(DecodeArgs da, int S, int32_t* part, int vec_out,
                                 hipStream_t stream) {
  if (da.G != 1 || S < 2 || S > kMaxSplits) return hipErrorInvalidValue;
  da.splits = S;
  da.part = part;
  hipError_t e = launch_skinny_t<TG, RB, NWK, SP, OUT>(da, stream);
  if (e != hipSuccess) return e;
  const GemmArgs ga{da.Wp[0], da.gamma[0], da.Ng[0], da.K, da.M, da.Xq, da.xs, da.xsum,
                    da.Y[0], 0, 0, vec_out, 0, S, part};
  const int64_t MN = (int64_t)ga.M * ga.N;
  const int64_t threads = ga.N % 4 == 0 ? MN / 4 : MN;
  k_splitk_reduce<OUT><<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream>>>(ga);
  return hipGetLastError();
}

// Where the skinny kernel takes a projection (or a group of them sharing the
// activations), `rows` being all output rows, each projection's rounded up
// to 16.  Timed on MI355X against the matrix decode and the GEMM on the 3B,
// 7B and 70B projections:
//   2-7 tokens: the matrix decode keeps more weight loads in flight on
//     narrow outputs (< 384 row blocks), and at 2 tokens on matrices of
//     less than 2^27 weights;
//   33-64 tokens: up to K = 8192 (8192 <- 8192 at 64 tokens: 13.7 us
//     against 16.5 us for the GEMM; 28672 <- 8192: 23.7 against 36.7 us);
//     longer K takes the GEMM unless the K-split skinny kernel applies.
inline int64_t group_rows(int G, const int64_t* N) {
  int64_t rows = 0;
  for (int g = 0; g < G; ++g) rows += 16 * ((N[g] + 15) / 16);
  return rows;
}

inline bool skinny_ok(int64_t M, int64_t rows, int64_t K) {
  if (K % 64 != 0 || M < 2 || M > 64) return false;
  if (M > 32) return K <= 8192;
  if (M >= 8) return true;
  if (rows < 16 * 384) return false;
  return M > 2 || rows * K >= (int64_t(1) << 27);
}

// About 256 workgroups of 8 waves: 4 row blocks of 2 waves on wide outputs
// (>= 640 row blocks), 2 of 4 waves on mid ones, 1 of 4 waves on narrow
// ones (each wave of a row block takes a quarter or half of every chunk).
// Rings of 3 stages, 2 above 16 tokens (LDS).
template <int TG, int OUT>
hipError_t launch_skinny_tg(const DecodeArgs& da, int nrb, hipStream_t stream) {
  constexpr int SP = TG == 1 ? 3 : 2;
  if (nrb >= 640) return launch_skinny_t<TG, 4, 2, SP, OUT>(da, stream);
  if (nrb >= 384) return launch_skinny_t<TG, 2, 4, SP, OUT>(da, stream);
  return launch_skinny_t<TG, 1, 4, SP, OUT>(da, stream);
}

template <int OUT>
hipError_t launch_skinny(const DecodeArgs& da, hipStream_t stream) {
  const int nrb = decode_rows(da) / 16;
  if (da.M <= 16) return launch_skinny_tg<1, OUT>(da, nrb, stream);
  if (da.M <= 32) {
    // 17-32 tokens on up to 512 row blocks: two halves of 16 tokens, each
    // workgroup taking twice the rows (the TS form, as at 33-64 tokens
    // below).  Timed at 17 / 24 / 32 tokens: 4096 <- 4096 4.76 / 4.88 / 4.92
    // against 5.31 / 5.59 / 5.73 us, 8192 <- 8192 8.86 / 8.99 / 9.05 against
    // 9.00 / 9.70 / 10.06 us (identical output bytes).
    if (da.M > 16 && nrb <= 512) {
      if (nrb >= 384) return launch_skinny_ts_t<1, 4, 2, 3, OUT>(da, stream);
      return launch_skinny_ts_t<1, 2, 4, 3, OUT>(da, stream);
    }
    return launch_skinny_tg<2, OUT>(da, nrb, stream);
  }
  // 33-64 tokens, one workgroup per CU.  Up to 512 row blocks: the tokens in
  // two halves of 32 (the TS form), each workgroup taking twice the rows of
  // one half, so that a CU takes in half the activations.  Timed at 33 / 48
  // / 64 tokens (bf16 out, rotated weights): 4096 <- 4096 7.13 / 7.14 / 7.53
  // against 8.23 / 8.40 / 8.83 us for all 64 tokens per workgroup, 8192 <-
  // 8192 10.83 / 10.87 / 11.22 against 12.78 / 13.05 / 13.87 us.  Wider
  // outputs keep all tokens per workgroup (11008 rows: 9.83 / 9.84 / 10.04
  // split against 9.57 / 10.09 / 10.57 us; 28672 rows: 29.1-29.7 split
  // against 25.5-27.7 us): as many row blocks per workgroup as keep the
  // launch to one round of at most 256 workgroups, 2 waves per row block,
  // and 8 one-wave row blocks past 1024 row blocks (at 64 tokens 11008 rows
  // 10.3 us at 3 row blocks, 16.6 at 2 in two rounds; 28672 rows 23.7 us at 8
  // one-wave row blocks, 29.5 at 4 of 2 waves in two rounds).
  if (nrb <= 512) {
    if (nrb > 128) return launch_skinny_ts_t<2, 4, 2, 2, OUT>(da, stream);
    return launch_skinny_ts_t<2, 2, 2, 2, OUT>(da, stream);
  }
  if (nrb > 1024) return launch_skinny_t<4, 8, 1, 2, OUT>(da, stream);
  if (nrb > 768) return launch_skinny_t<4, 4, 2, 2, OUT>(da, stream);
  return launch_skinny_t<4, 3, 2, 2, OUT>(da, stream);
}

// 17-64 tokens on one projection whose K is long against its rows (K >= 2 N,
// M K > 256 Ki): the skinny kernel with 4 row blocks per workgroup (8 at 33+
// tokens on 8192+ rows), so that more rows share each activation chunk, and
// K split S ways to keep about 256 workgroups; the partial sums are added
// exactly by k_splitk_reduce.  Timed on MI355X (bf16 out): 8192 <- 28672 at
// 64 tokens 25.5 us against 38.4 us for the GEMM, at 32 tokens 20.4 against
// 23.4 us for the unsplit skinny kernel; 4096 <- 11008 at 33-64 tokens
// 6-8 % faster than the GEMM, at 32 tokens 5 % faster than unsplit.  Wide
// projections (4096 -> 11008) and 16 tokens were slower split.
struct SkinnySplit {
  int tg, rb, s;   // token groups, row blocks per workgroup, K splits (s < 2: none)
};

inline SkinnySplit skinny_split_cfg(int64_t M, int64_t N, int64_t K) {
  SkinnySplit c{0, 0, 1};
  if (M < 17 || M > 64 || K % 64 != 0 || K < 2 * N || M * K <= 256 * 1024) return c;
  // 17-32 tokens on up to 512 row blocks: the token halves of launch_skinny
  // instead (no reduction launch).  Timed at 24 / 32 tokens: 4096 <- 11008
  // 8.05 / 8.48 against 9.55 / 9.74 us split, 8192 <- 28672 20.90 / 21.59
  // against 22.79 / 24.99 us (identical output bytes).
  if (M <= 32 && (N + 15) / 16 <= 512) return c;
  const int64_t nrb = (N + 15) / 16;
  c.tg = M <= 32 ? 2 : 4;
  c.rb = (c.tg == 4 && nrb >= 512) ? 8 : 4;
  const int64_t groups = (nrb + c.rb - 1) / c.rb;
  int s = (int)std::min<int64_t>(kMaxSplits, std::max<int64_t>(2, (256 + groups / 2) / groups));
  // two 512-wide chunks per split on average, and none empty: the kernel
  // gives split sp the chunks from sp * ceil(nch / s) on
  const int64_t nch = (K + 511) / 512;
  while (s >= 2 && (nch < 2 * s || (s - 1) * ((nch + s - 1) / s) >= nch)) --s;
  c.s = s;
  return c;
}

inline size_t skinny_split_workspace_bytes(const SkinnySplit& c, int64_t M, int64_t N) {
  return c.s < 2 ? 0 : (size_t)(((c.s * M * N * 4) + 255) / 256 * 256);
}

template <int OUT>
hipError_t launch_skinny_split(const SkinnySplit& c, const DecodeArgs& da, void* workspace,
                               hipStream_t stream) {
  const uintptr_t ya = reinterpret_cast<uintptr_t>(da.Y[0]);
  const int vec_out = (da.Ng[0] % 4 == 0) && (ya % (OUT == kOutBF16 ? 8 : 16) == 0);
  int32_t* part = reinterpret_cast<int32_t*>(workspace);
  if (c.tg == 2) return launch_skinny_split_t<2, 4, 2, 2, OUT>(da, c.s, part, vec_out, stream);
  if (c.rb == 8) return launch_skinny_split_t<4, 8, 2, 2, OUT>(da, c.s, part, vec_out, stream);
  return launch_skinny_split_t<4, 4, 2, 2, OUT>(da, c.s, part, vec_out, stream);
}

struct GemmCfg {
  int bm, bn;
  int splits;   // K splits (1: none)
};

template <bool A64, int OUT, int BM, int BN, int WM, int WN, int NS = 3, bool PF = false,
          int WPE = 1>
hipError_t launch_gemm_t(GemmArgs ga, hipStream_t stream) {
  ga.tiles_m = (ga.M + BM - 1) / BM;
  ga.tiles_n = (ga.N + BN - 1) / BN;
  if (ga.band <= 0 || ga.band > ga.tiles_n) ga.band = ga.tiles_n;
  if (ga.splits < 1) ga.splits = 1;
  if (ga.splits > kMaxSplits) return hipErrorInvalidValue;   // the reduction adds at most that many
  const int items = ga.tiles_m * ga.tiles_n * ga.splits;
  k_gemm<A64, OUT, BM, BN, WM, WN, NS, PF, WPE><<<dim3(items), dim3(kGemmThreads), 0, stream>>>(ga);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ga.splits == 1) return e;
  const int64_t MN = (int64_t)ga.M * ga.N;
  const int64_t threads = ga.N % 4 == 0 ? MN / 4 : MN;
  k_splitk_reduce<OUT><<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream>>>(ga);
  return hipGetLastError();
}

// 64 x 64 tiles up to 128 tokens (more workgroups to fill the chip), else
// 128 x 128.  At most 128 tiles (a half-empty chip): K split up to 4 ways,
// each split keeping at least 4 steps of 128 and the partial sums (written
// and read back: 8 S M N bytes) costing no more traffic than the packed
// weights (N K / 4 bytes): S <= K / (16 M).  Timed on MI355X: splitting the
// 172-tile shapes (N = 11008, M <= 128) loses to the reduction's cost.
inline GemmCfg gemm_cfg(int M, int N, int K) {
  GemmCfg c{128, 128, 1};
  if (M <= 128) c = {64, 64, 1};
  // 1024+ tokens: 128 x 256 tiles at two waves per SIMD, 2 x 2 waves (a 64 x
  // 128 sub-tile each).  Timed on MI355X (same process, three runs): ffn-70b
  // at 1024 tokens, 8192 -> 28672 in 197-200 us against 200-204 with the
  // four waves side by side along N, and 28672 -> 8192 in 191-199 against
  // 197-201 with 128 x 128 tiles; prefill-7b (2048 x 11008 x 4096) the same
  // within 0.5 %.
  else if (M >= 1024) c = {128, 256, 1};
  const int tiles = ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
  const int nk = K / kGBK;
  if (tiles <= 128) c.splits = max(1, min(kMaxSplits, min(nk / 4, K / (16 * M))));
  return c;
}

// Partial accumulators of the split GEMM, 256-byte aligned.
inline size_t gemm_workspace_bytes(const GemmCfg& c, int64_t M, int64_t N) {
  if (c.splits <= 1) return 0;
  return (size_t)(((c.splits * M * N * 4) + 255) / 256 * 256);
}

template <bool A64, int OUT>
hipError_t launch_gemm(const GemmCfg& c, GemmArgs ga, hipStream_t stream) {
  ga.splits = c.splits;
  if (c.bm == 128 && c.bn == 128) return launch_gemm_t<A64, OUT, 128, 128, 2, 2, 3>(ga, stream);
  if (c.bm == 128 && c.bn == 256)
    return launch_gemm_t<A64, OUT, 128, 256, 2, 2, 3, false, 2>(ga, stream);
  // 64 x 64 tiles run one workgroup per CU (a single wave per SIMD), so the
  // fragment reads are pipelined a step ahead there (timed 5-7 % faster);
  // at 128 x 128 two workgroups per CU already hide them.
  if (c.bm == 64 && c.bn == 64) return launch_gemm_t<A64, OUT, 64, 64, 2, 2, 4, true>(ga, stream);
  return hipErrorInvalidValue;
}

// Decode (M <= 16) over every projection of `da` in one launch.
template <bool A64, int OUT>
hipError_t decode_grouped(const DecodeArgs& da, hipStream_t stream) {
  // One token and rows of at most 64 pieces (one per lane): the vector-ALU
  // kernel, 4 rows per wave (timed 12-18 % faster than the matrix kernel on
  // the 3B and 7B single-token shapes, and 1-4 % faster than 2 rows).
  if (da.M == 1 && A64 && da.K <= 64 * 64) return launch_decode_dot_t<OUT, 4, 1>(da, stream);
  return launch_decode<A64, OUT>(decode_cfg(da.M, decode_rows(da), da.K, false), da, stream);
}

template <bool A64, int OUT>
hipError_t dispatch(const uint8_t* Wp, const float* gamma, int N, int K, const int8_t* Xq,
                    const float* xs, const int32_t* xsum, int M, void* Y, void* workspace,
                    hipStream_t stream) {
  // 2: bf16 rows through LDS with 16-byte stores; 1: 4-wide stores (split-K
  // reduction); 0: scalar.
  const uintptr_t ya = reinterpret_cast<uintptr_t>(Y);
  int vec_out = (N % 4 == 0) && (ya % (OUT == kOutBF16 ? 8 : 16) == 0);
  if (OUT == kOutBF16 && N % 8 == 0 && ya % 16 == 0) vec_out = 2;
  const GemmCfg c = gemm_cfg(M, N, K);
  GemmArgs ga{Wp, gamma, N, K, M, Xq, xs, xsum, Y, 0, 0, vec_out, 16, 1,
              reinterpret_cast<int32_t*>(workspace)};
  return launch_gemm<A64, OUT>(c, ga, stream);
}

template <int OUT>
hipError_t dispatch_out(const uint8_t* Wp, const float* gamma, int N, int K, const int8_t* Xq,
                        const float* xs, const int32_t* xsum, int M, void* Y, void* workspace,
                        hipStream_t stream) {
  if (K % 64 == 0) return dispatch<true, OUT>(Wp, gamma, N, K, Xq, xs, xsum, M, Y, workspace, stream);
  return dispatch<false, OUT>(Wp, gamma, N, K, Xq, xs, xsum, M, Y, workspace, stream);
}

}  // namespace

namespace {
// Workspace of one projection on the GEMM (0 where the shape takes another kernel).
size_t gemm_path_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 16 || skinny_ok(M, 16 * ((N + 15) / 16), K)) return 0;
  return gemm_workspace_bytes(gemm_cfg((int)M, (int)N, (int)K), M, N);
}
}  // namespace

size_t forward_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const SkinnySplit ss = skinny_split_cfg(M, N, K);
  if (ss.s >= 2) return skinny_split_workspace_bytes(ss, M, N);
  return gemm_path_workspace_bytes(M, N, K);
}

// A group splits no projection's K in the skinny kernel: it runs as one
// skinny or decode launch, or as one GEMM per projection.
size_t forward_grouped_workspace_bytes(int64_t M, int G, const int64_t* N, int64_t K) {
  if (G == 1) return forward_workspace_bytes(M, N[0], K);
  if (M <= 16 || skinny_ok(M, group_rows(G, N), K)) return 0;   // one launch over the group
  size_t need = 0;
  for (int g = 0; g < G; ++g) need = std::max(need, gemm_path_workspace_bytes(M, N[g], K));
  return need;
}

namespace {
DecodeArgs decode_args_group(int G, const uint8_t* const* Wp, const float* const* gamma,
                             const int64_t* N, int K, int M, void* const* Y) {
  DecodeArgs da{};
  for (int g = 0; g < G; ++g) {
    da.Wp[g] = Wp[g];
    da.gamma[g] = gamma[g];
    da.Ng[g] = (int)N[g];
    da.Y[g] = Y[g];
  }
  da.G = G;
  da.K = K;
  da.M = M;
  return da;
}

template <int OUT>
hipError_t forward_grouped_out(int G, const uint8_t* const* Wp, const float* const* gamma,
                               const int64_t* N, int K, const int8_t* Xq, const float* xs,
                               const int32_t* xsum, int M, void* const* Y, void* workspace,
                               hipStream_t stream) {
  DecodeArgs da = decode_args_group(G, Wp, gamma, N, K, M, Y);
  da.Xq = Xq;
  da.xs = xs;
  da.xsum = xsum;
  // One projection with a long K: the K-split skinny kernel.
  const SkinnySplit ss = G == 1 ? skinny_split_cfg(M, N[0], K) : SkinnySplit{0, 0, 1};
  if (ss.s >= 2) return launch_skinny_split<OUT>(ss, da, workspace, stream);
  // Every projection of the group in one launch where the skinny kernel or
  // the decode takes the shape.
  if (skinny_ok(M, decode_rows(da), K)) return launch_skinny<OUT>(da, stream);
  if (M <= 16)
    return K % 64 == 0 ? decode_grouped<true, OUT>(da, stream)
                       : decode_grouped<false, OUT>(da, stream);
  // GEMM shapes: one projection after another (the workspace is reused in
  // stream order).
  for (int g = 0; g < G; ++g) {
    const hipError_t e = dispatch_out<OUT>(Wp[g], gamma[g], (int)N[g], K, Xq, xs, xsum, M, Y[g],
                                           workspace, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}
}  // namespace

hipError_t launch_forward_grouped(int G, const uint8_t* const* W_packed,
                                  const float* const* gamma, const int64_t* N, int64_t K,
                                  const int8_t* X_q, const float* x_scale, const int32_t* x_sum,
                                  int64_t M, void* const* Y, int y_dtype, void* workspace,
                                  hipStream_t stream) {
  const int k = (int)K, m = (int)M;
  switch (y_dtype) {
    case kOutF32:
      return forward_grouped_out<kOutF32>(G, W_packed, gamma, N, k, X_q, x_scale, x_sum, m, Y,
                                          workspace, stream);
    case kOutBF16:
      return forward_grouped_out<kOutBF16>(G, W_packed, gamma, N, k, X_q, x_scale, x_sum, m, Y,
                                           workspace, stream);
    default:
      return forward_grouped_out<kOutI32>(G, W_packed, gamma, N, k, X_q, x_scale, x_sum, m, Y,
                                          workspace, stream);
  }
}

hipError_t launch_forward(const uint8_t* W_packed, const float* gamma, int64_t N, int64_t K,
                          const int8_t* X_q, const float* x_scale, const int32_t* x_sum,
                          int64_t M, void* Y, int y_dtype, void* workspace, hipStream_t stream) {
  return launch_forward_grouped(1, &W_packed, &gamma, &N, K, X_q, x_scale, x_sum, M, &Y, y_dtype,
                                workspace, stream);
}

}  // namespace bl

namespace bl {

// Quantiser outputs (when the caller passes none), then the projection's
// own workspace.
inline size_t quant_region_bytes(int64_t M, int64_t K) {
  return (size_t)(((M * K + 255) / 256) * 256 + ((8 * M + 255) / 256) * 256);
}

// The fused launch for a decode group, or none (kind < 0).
inline DecodeCfg fused_cfg(int64_t M, int G, const int64_t* N, int64_t K) {
  DecodeCfg c{};
  c.am = -1;
  if (M > 16) return c;
  int rows = 0;
  for (int g = 0; g < G; ++g) rows += 16 * (int)((N[g] + 15) / 16);
  return decode_cfg((int)M, rows, (int)K, true);
}

// One token with K a multiple of 64 up to 16384 (12288 with the
// normalisation): the vector-ALU decode quantises in place (the workgroup
// converts the row once into LDS), one launch and no workspace; Q =
// ceil(K / 4096) pieces per lane.  4 rows per wave and 4 waves per
// workgroup, except at Q = 3, 4 without the normalisation: 2 rows per wave
// and 8 waves, timed faster there (3200 <- 8640: 5.8 vs 6.3 us; 4096 <-
// 11008: 6.6 vs 6.9 us; 8192 <- 12288: 9.3-9.8 vs 10.0-10.4 us) and no
// faster at Q = 1, 2; and at Q = 2 without the normalisation on 16384+
// output rows, 4 rows per wave and 8 waves (half as many workgroups, each
// converting the row once: 28672 <- 8192 15.8 vs 16.4 us, 16384 <- 8192
// 10.1 vs 11.0 us; 8 waves were no faster at Q = 1).  At Q = 4 (8192 <- 16384) it takes 12.3-12.7 us
// against 14.6 us for the matrix decode with the quantiser in its prologue;
// beyond (Q = 5..7: 4096 <- 20480, 8192 <- 28672) it no longer wins.  With
// the normalisation 4 rows per wave and 4 waves throughout (its fp32 row and
// gain fill the registers at Q = 4, so it stops at Q = 3).
constexpr int kDotFuseRows = 4;   // rows per wave in that mode
constexpr int kDotFuseWaves = 4;  // waves per workgroup in that mode
constexpr int kDotFuseMaxQ = 4;
constexpr int kDotFuseNormMaxQ = 3;
inline bool fused_dot(int64_t M, int64_t K, bool norm) {
  return M == 1 && K % 64 == 0 && K <= 64 * 64 * (norm ? kDotFuseNormMaxQ : kDotFuseMaxQ);
}

namespace {
template <int OUT, bool NORM>
hipError_t fused_dot_out(const DecodeArgs& da, hipStream_t stream) {
  const int q = (da.K + 64 * 64 - 1) / (64 * 64);
  if (q <= 1) return launch_decode_dot_t<OUT, kDotFuseRows, 1, kDotFuseBlock, kDotFuseWaves, NORM>(da, stream);
  if (q == 2) {
    if (!NORM && decode_rows(da) >= 16384)
      return launch_decode_dot_t<OUT, kDotFuseRows, 2, kDotFuseBlock, 8, false>(da, stream);
    return launch_decode_dot_t<OUT, kDotFuseRows, 2, kDotFuseBlock, kDotFuseWaves, NORM>(da, stream);
  }
  if constexpr (NORM) {
    return launch_decode_dot_t<OUT, kDotFuseRows, 3, kDotFuseBlock, kDotFuseWaves, true>(da, stream);
  } else {
    if (q == 3) return launch_decode_dot_t<OUT, 2, 3, kDotFuseBlock, 8, false>(da, stream);
    return launch_decode_dot_t<OUT, 2, 4, kDotFuseBlock, 8, false>(da, stream);
  }
}
template <int OUT>
hipError_t fused_dot_norm(const DecodeArgs& da, hipStream_t stream) {
  return da.norm_g ? fused_dot_out<OUT, true>(da, stream) : fused_dot_out<OUT, false>(da, stream);
}
}  // namespace

// The matrix decode with the quantiser in its prologue: one or two tokens,
// where the skinny kernel does not take the shape.  Timed against the
// quantiser launch + the unfused decode: faster at one token (70B down,
// 8192 <- 28672: 19.0 vs 24.2 us) and two (3200 <- 8640: 7.7 vs 9.0 us);
// slower from four tokens on (4096 <- 4096: 7.7 vs 7.1 us at 4, 8.3 vs
// 7.3 us at 7), where every workgroup's re-quantisation of the fp32 rows
// outweighs the saved launch.
inline bool afuse(int64_t M, int G, const int64_t* N, int64_t K) {
  return M <= 2 && fused_cfg(M, G, N, K).am == kAFuse && !skinny_ok(M, group_rows(G, N), K);
}

// One projection, one token, no normalisation, at least 2^25 weights: the
// persistent launch (k_stream) instead of the fused vector-ALU or matrix
// decode.  Timed on MI355X with graph replay over rotated weight copies
// (identical output bytes): 8192 -> 28672 12.6 against 14.4 us, 28672 ->
// 8192 15.8 against 19.0 us, 4096 <-> 11008 6.07 / 6.18 against 6.23 / 6.66
// us; below the threshold it was slower (4096 -> 4096 3.99 against 3.41 us)
// or even (8640 -> 3200 5.43 against 5.36 us), and for q/k/v as one grouped
// call it gained nothing in the step (5.95 against 5.69 us).
constexpr int64_t kStreamSingleMinWeights = int64_t(1) << 25;

inline bool stream_single(int64_t M, int G, const int64_t* N, int64_t K) {
  if (M != 1 || G != 1) return false;
  return N[0] * K >= kStreamSingleMinWeights && stream_multi_ok(1, 1, N, &K);
}

hipError_t launch_stream_shared(int G, const uint8_t* const* W_packed, const float* const* gamma,
                                const int64_t* N, int64_t K, const float* X, void* const* Y,
                                int y_dtype, int8_t* X_q_out, float* x_scale_out,
                                int32_t* x_sum_out, hipStream_t stream);

// norm: RMS normalisation first; the single-token vector-ALU prologue fuses
// it, the multi-token matrix prologue does not (two launches there).
size_t forward_f32_grouped_workspace_bytes(int64_t M, int G, const int64_t* N, int64_t K,
                                           bool norm) {
  if (!norm && stream_single(M, G, N, K)) return 0;
  if (fused_dot(M, K, norm) || (!norm && afuse(M, G, N, K))) return 0;
  return quant_region_bytes(M, K) + forward_grouped_workspace_bytes(M, G, N, K);
}

size_t forward_f32_workspace_bytes(int64_t M, int64_t N, int64_t K, bool norm) {
  return forward_f32_grouped_workspace_bytes(M, 1, &N, K, norm);
}

namespace {
template <int OUT>
hipError_t fused_out(const DecodeCfg& c, const DecodeArgs& da, hipStream_t stream) {
  if (da.K % 64 == 0) return launch_decode<true, OUT>(c, da, stream);
  return launch_decode<false, OUT>(c, da, stream);
}
}  // namespace

hipError_t launch_forward_f32_grouped(int G, const uint8_t* const* W_packed,
                                      const float* const* gamma, const int64_t* N, int64_t K,
                                      const float* X, const float* norm_g, int64_t M,
                                      void* const* Y, int y_dtype, int8_t* X_q_out,
                                      float* x_scale_out, int32_t* x_sum_out, void* workspace,
                                      hipStream_t stream) {
  if (norm_g == nullptr && stream_single(M, G, N, K))
    return launch_stream_shared(G, W_packed, gamma, N, K, X, Y, y_dtype, X_q_out, x_scale_out,
                                x_sum_out, stream);
  if (fused_dot(M, K, norm_g != nullptr)) {
    DecodeArgs da = decode_args_group(G, W_packed, gamma, N, (int)K, (int)M, Y);
    da.X = X;
    da.Xq_out = X_q_out;
    da.xs_out = x_scale_out;
    da.xsum_out = x_sum_out;
    da.norm_g = norm_g;
    switch (y_dtype) {
      case kOutF32: return fused_dot_norm<kOutF32>(da, stream);
      case kOutBF16: return fused_dot_norm<kOutBF16>(da, stream);
      default: return fused_dot_norm<kOutI32>(da, stream);
    }
  }
  if (norm_g == nullptr && afuse(M, G, N, K)) {
    const DecodeCfg c = fused_cfg(M, G, N, K);
    DecodeArgs da = decode_args_group(G, W_packed, gamma, N, (int)K, (int)M, Y);
    da.X = X;
    da.Xq_out = X_q_out;
    da.xs_out = x_scale_out;
    da.xsum_out = x_sum_out;
    switch (y_dtype) {
      case kOutF32: return fused_out<kOutF32>(c, da, stream);
      case kOutBF16: return fused_out<kOutBF16>(c, da, stream);
      default: return fused_out<kOutI32>(c, da, stream);
    }
  }
  // Two launches: quantise once into the caller's output buffers (or the
  // workspace), then every projection.
  int8_t* xq = X_q_out;
  float* xs = x_scale_out;
  int32_t* xsum = x_sum_out;
  char* w = reinterpret_cast<char*>(workspace);
  if (xq == nullptr) {
    xq = reinterpret_cast<int8_t*>(w);
    xs = reinterpret_cast<float*>(w + ((M * K + 255) / 256) * 256);
    xsum = reinterpret_cast<int32_t*>(xs + M);
  }
  // The projections' workspace follows the quantiser region (present in the
  // size query in both cases).
  void* fws = w ? w + quant_region_bytes(M, K) : nullptr;
  hipError_t e = norm_g ? launch_rmsnorm_quant(X, norm_g, M, K, xq, xs, xsum, stream)
                        : launch_quant(X, M, K, xq, xs, xsum, stream);
  if (e != hipSuccess) return e;
  return launch_forward_grouped(G, W_packed, gamma, N, K, xq, xs, xsum, M, Y, y_dtype, fws,
                                stream);
}

int forward_kernel(int entry, int64_t M, int G, const int64_t* N, int64_t K) {
  constexpr int kFused = 16;
  if (entry != 0) {
    if (entry == 1 && stream_single(M, G, N, K)) return kKernelStream | kFused;
    if (fused_dot(M, K, entry == 2)) return kKernelDecodeDot | kFused;
    if (entry == 1 && afuse(M, G, N, K)) return kKernelDecode | kFused;
  }
  if (G == 1 && skinny_split_cfg(M, N[0], K).s >= 2) return kKernelSkinny;
  if (skinny_ok(M, group_rows(G, N), K)) return kKernelSkinny;
  if (M <= 16) return M == 1 && K % 64 == 0 && K <= 64 * 64 ? kKernelDecodeDot : kKernelDecode;
  return kKernelGemm;
}

hipError_t launch_forward_f32(const uint8_t* W_packed, const float* gamma, int64_t N, int64_t K,
                              const float* X, const float* norm_g, int64_t M, void* Y,
                              int y_dtype, int8_t* X_q_out, float* x_scale_out,
                              int32_t* x_sum_out, void* workspace, hipStream_t stream) {
  return launch_forward_f32_grouped(1, &W_packed, &gamma, &N, K, X, norm_g, M, &Y, y_dtype,
                                    X_q_out, x_scale_out, x_sum_out, workspace, stream);
}

}  // namespace bl

namespace bl {

// ---- several projections with their own activations (stream.hpp) ---------

namespace {

// Compute units of the current device (workgroups of the persistent launch),
// cached per device.
std::atomic<int> g_cus[64];

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = g_cus[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v <= 0)
      v = 256;
    g_cus[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// Launch shape (timed on MI355X over the 3B, 7B and 70B single-token steps,
// all projections in one launch): 4 rows per step, loads 1 step ahead, 8
// waves, one workgroup per CU.  Loads 1 step ahead against 2: 70B 8192 ->
// 28672 with 28672 -> 8192 22.08 against 22.13 us, 7B 7.99 against 8.89 us,
// 3B 6.26 against 7.25 us (at 3B and 7B sizes a wave has 2-4 steps, which a
// ring of two runs as whole unguarded rounds); 2 rows per step, or deeper
// rings, were slower.  Against two fused single-projection calls on the
// earlier kernels: 70B 22.1 against 33.6 us.  (Single projections take this
// launch from 2^25 weights: stream_single.)
constexpr int kStreamR = 4, kStreamP = 1, kStreamWV = 8;

StreamArgs stream_args(int G, const uint8_t* const* Wp, const float* const* gamma,
                       const int64_t* N, const int64_t* K, const float* const* X,
                       void* const* Y) {
  StreamArgs sa{};
  sa.G = G;
  for (int g = 0; g < G; ++g) {
    sa.rec[g].Wp = Wp[g];
    sa.rec[g].X = X[g];
    sa.rec[g].N = (int)N[g];
    sa.rec[g].K = (int)K[g];
    sa.gamma[g] = gamma[g];
    sa.Y[g] = Y[g];
  }
  return sa;
}

template <int OUT, int KJ>
hipError_t launch_stream_kj(const StreamArgs& sa, int nwg, hipStream_t stream) {
  if (sa.xq_out != nullptr)
    k_stream<OUT, kStreamR, kStreamP, kStreamWV, KJ, true>
        <<<dim3(nwg), dim3(kStreamWV * kWave), 0, stream>>>(sa);
  else
    k_stream<OUT, kStreamR, kStreamP, kStreamWV, KJ, false>
        <<<dim3(nwg), dim3(kStreamWV * kWave), 0, stream>>>(sa);
  return hipGetLastError();
}

template <int OUT>
hipError_t launch_stream_out(const StreamArgs& sa, int nwg, int64_t maxK, hipStream_t stream) {
  // fp32 values per thread held for the quantiser: 4 KJ per thread, 512 threads
  if (maxK <= 8192) return launch_stream_kj<OUT, 4>(sa, nwg, stream);
  if (maxK <= 16384) return launch_stream_kj<OUT, 8>(sa, nwg, stream);
  return launch_stream_kj<OUT, 16>(sa, nwg, stream);
}

}  // namespace

bool stream_multi_ok(int64_t M, int G, const int64_t* N, const int64_t* K) {
  if (M != 1 || G < 1 || G > kStreamMaxProj) return false;
  for (int g = 0; g < G; ++g)
    if (K[g] % 64 != 0 || K[g] > kStreamMaxK || N[g] < 1) return false;
  // the share of rows per workgroup must fit the LDS accumulators: planned
  // for the smallest GPU the library takes (64 CUs)
  StreamArgs sa{};
  sa.G = G;
  for (int g = 0; g < G; ++g) {
    sa.rec[g].N = (int)N[g];
    sa.rec[g].K = (int)K[g];
  }
  return stream_plan(sa, 64, kStreamR) > 0;
}

// Shapes the persistent launch does not take: where no projection has a
// single-launch fused path, one quantiser launch for every input, then one
// projection launch each (G - 1 launches fewer than a bitlinear_forward_f32
// per projection); else one bitlinear_forward_f32 per projection.
inline bool multi_quant_once(int64_t M, int G, const int64_t* N, const int64_t* K) {
  if (G < 2 || G > kQuantMaxMulti) return false;
  for (int g = 0; g < G; ++g)
    if (fused_dot(M, K[g], false) || afuse(M, 1, &N[g], K[g])) return false;
  return true;
}

size_t forward_f32_multi_workspace_bytes(int64_t M, int G, const int64_t* N, const int64_t* K) {
  if (stream_multi_ok(M, G, N, K)) return 0;
  size_t need = 0;
  if (multi_quant_once(M, G, N, K)) {
    // every input's quantiser region, then the largest projection workspace
    size_t q = 0;
    for (int g = 0; g < G; ++g) {
      q += quant_region_bytes(M, K[g]);
      need = std::max(need, forward_grouped_workspace_bytes(M, 1, &N[g], K[g]));
    }
    return q + need;
  }
  for (int g = 0; g < G; ++g)
    need = std::max(need, forward_f32_workspace_bytes(M, N[g], K[g], false));
  return need;
}

hipError_t launch_forward_f32_multi(int G, const uint8_t* const* W_packed,
                                   const float* const* gamma, const int64_t* N, const int64_t* K,
                                   const float* const* X, int64_t M, void* const* Y, int y_dtype,
                                   void* workspace, hipStream_t stream) {
  if (stream_multi_ok(M, G, N, K)) {
    StreamArgs sa = stream_args(G, W_packed, gamma, N, K, X, Y);
    const int nwg = stream_plan(sa, std::max(device_cus(), 64), kStreamR);
    if (nwg <= 0) return hipErrorInvalidValue;
    int64_t maxK = 0;
    for (int g = 0; g < G; ++g) maxK = std::max(maxK, K[g]);
    switch (y_dtype) {
      case kOutF32: return launch_stream_out<kOutF32>(sa, nwg, maxK, stream);
      case kOutBF16: return launch_stream_out<kOutBF16>(sa, nwg, maxK, stream);
      default: return launch_stream_out<kOutI32>(sa, nwg, maxK, stream);
    }
  }
  if (multi_quant_once(M, G, N, K)) {
    char* w = reinterpret_cast<char*>(workspace);
    int8_t* xq[kQuantMaxMulti];
    float* xs[kQuantMaxMulti];
    int32_t* xsum[kQuantMaxMulti];
    for (int g = 0; g < G; ++g) {
      xq[g] = reinterpret_cast<int8_t*>(w);
      xs[g] = reinterpret_cast<float*>(w + ((M * K[g] + 255) / 256) * 256);
      xsum[g] = reinterpret_cast<int32_t*>(xs[g] + M);
      w += quant_region_bytes(M, K[g]);
    }
    hipError_t e = launch_quant_multi(G, X, M, K, xq, xs, xsum, stream);
    for (int g = 0; g < G && e == hipSuccess; ++g)
      e = launch_forward_grouped(1, &W_packed[g], &gamma[g], &N[g], K[g], xq[g], xs[g], xsum[g], M,
                                 &Y[g], y_dtype, w, stream);
    return e;
  }
  for (int g = 0; g < G; ++g) {
    const hipError_t e = launch_forward_f32(W_packed[g], gamma[g], N[g], K[g], X[g], nullptr, M,
                                            Y[g], y_dtype, nullptr, nullptr, nullptr, workspace,
                                            stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_stream_shared(int G, const uint8_t* const* W_packed, const float* const* gamma,
                                const int64_t* N, int64_t K, const float* X, void* const* Y,
                                int y_dtype, int8_t* X_q_out, float* x_scale_out,
                                int32_t* x_sum_out, hipStream_t stream) {
  const float* Xs[kStreamMaxProj];
  int64_t Ks[kStreamMaxProj];
  for (int g = 0; g < G; ++g) {
    Xs[g] = X;
    Ks[g] = K;
  }
  StreamArgs sa = stream_args(G, W_packed, gamma, N, Ks, Xs, Y);
  sa.xq_out = X_q_out;
  sa.xs_out = x_scale_out;
  sa.xsum_out = x_sum_out;
  const int nwg = stream_plan(sa, std::max(device_cus(), 64), kStreamR);
  if (nwg <= 0) return hipErrorInvalidValue;
  switch (y_dtype) {
    case kOutF32: return launch_stream_out<kOutF32>(sa, nwg, K, stream);
    case kOutBF16: return launch_stream_out<kOutBF16>(sa, nwg, K, stream);
    default: return launch_stream_out<kOutI32>(sa, nwg, K, stream);
  }
}

}  // namespace bl
