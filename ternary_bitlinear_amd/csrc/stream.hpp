// Single-token decode as one persistent launch over one or more projections
// (each with its own activations, K and N), the quantiser optionally in the
// prologue.
//
// Page "BitNet b1.58: Mathematical Foundations ..." (llms.blog), section 2,
// "The Linear Transformation and Rescaling" (acc = x~ . W~ in int32, then the
// rescale by gamma beta / 127) and section 4, "Memory Bandwidth and Latency
// Bounds": at one token the projection reads every packed weight once and
// does a handful of integer operations per byte, so its time is the time to
// stream the weights.  This kernel is shaped for that stream:
//
//   - One workgroup per CU for the whole launch (no second round of
//     workgroups, no tail), each owning a contiguous range of row groups of
//     one projection (workgroups are shared out in proportion to the
//     projections' bytes).  The quantiser (absmax, factor, codes; the same
//     per-element arithmetic as the standalone quantiser), or the copy of
//     pre-quantised activations, runs once per workgroup into LDS, while the
//     first weight loads are already in flight.
//   - The workgroup's work is a list of steps (row group of R rows, chunk of
//     4096 weights); wave w takes a contiguous share of it.  A step loads one
//     16-byte piece of each of the R rows per lane (whole 1 KB lines per
//     wave, with the non-temporal hint: the weights are read once), reads the lane's 64 activations once from LDS for all R rows, and
//     multiplies on the vector ALU (v_dot4_i32_i8 on codes expanded in
//     registers).  Loads run P steps ahead through P + 1 register buffers, so
//     the next loads go out before the current step computes.
//   - A wave's partial sums of a row group are reduced across the wave (DPP)
//     and added into LDS with integer atomics (exact and order-free) whenever
//     its share leaves the row group; after one barrier the workgroup stores
//     its rows with the epilogue.
//
// Codes are c = W~ + 1 (BLT2-v1); the kernel forms sum_k c_k x~_k and
// subtracts sum_k x~_k, as the other projection kernels do.
#pragma once

#include "common.hpp"

namespace bl {

constexpr int kStreamMaxProj = 4;

struct StreamProj {
  const uint8_t* Wp;
  const float* gamma;
  void* Y;
  int N, K;
  const int8_t* Xq;        // pre-quantised activations [K] (unfused), x_scale, x_sum
  const float* xs;
  const int32_t* xsum;
  const float* X;          // fp32 activations [K] (fused)
  int8_t* Xq_out;          // fused: optional quantiser outputs (written by one workgroup)
  float* xs_out;
  int32_t* xsum_out;
  int wg0, nwg;            // this projection's first workgroup and workgroup count
};

struct StreamArgs {
  StreamProj p[kStreamMaxProj];
  int G;
};

// The LDS layout of the kernel: activations (K bytes, padded) and a 64-byte
// zero slot, then the row accumulators of the workgroup, then reduction slots.
constexpr int kStreamMaxK = 32768;
constexpr int kStreamMaxRowsWg = 4096;

template <int OUT, int R, int P, int WV, int KJ>
__global__ __launch_bounds__(WV * kWave) void k_stream(StreamArgs sa) {
  constexpr int NB = P + 1;
  constexpr int T = WV * kWave;
  __shared__ __attribute__((aligned(16))) int8_t xl[kStreamMaxK + 64];
  __shared__ int32_t acc_l[kStreamMaxRowsWg];
  __shared__ uint32_t s_red[2][WV];

  // this workgroup's projection: branch-free pick over the table
  const int b = blockIdx.x;
  int gsel = 0;
#pragma unroll
  for (int i = 1; i < kStreamMaxProj; ++i) gsel += (i < sa.G && b >= sa.p[i].wg0) ? 1 : 0;
  StreamProj pj = sa.p[0];
#pragma unroll
  for (int i = 1; i < kStreamMaxProj; ++i)
    if (gsel == i) pj = sa.p[i];
  const int N = pj.N, K = pj.K;
  const int lw = b - pj.wg0;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int npieces = K / 64;
  const int Q = (npieces + 63) / 64;                 // chunks of 4096 weights per row
  const int ngroups = (N + R - 1) / R;
  const int g0 = (int)((int64_t)lw * ngroups / pj.nwg);
  const int g1 = (int)((int64_t)(lw + 1) * ngroups / pj.nwg);
  const int S = (g1 - g0) * Q;                       // steps of the workgroup
  const int s0 = (int)((int64_t)wave * S / WV);
  const int s1 = (int)((int64_t)(wave + 1) * S / WV);
  const int kbytes = K / 4;

  // fused: the fp32 row first (its loads must not queue behind the weights')
  float4 xv[KJ > 0 ? KJ : 1];
  if constexpr (KJ > 0) {
    const float4* src = reinterpret_cast<const float4*>(pj.X);
    const int K4 = K / 4;
#pragma unroll
    for (int j = 0; j < KJ; ++j) {
      const int i = threadIdx.x + T * j;
      xv[j] = src[i < K4 ? i : 0];
    }
  } else {
    const i32x4* src = reinterpret_cast<const i32x4*>(pj.Xq);
    for (int i = threadIdx.x; i < K / 16; i += T)
      reinterpret_cast<i32x4*>(xl)[i] = src[i];
  }

  uint4 wq[NB][R];
  auto fill = [&](int bf, int s) {
    s = min(s, s1 - 1);
    const int gl = s / Q, c = s - gl * Q;
    const int p = 64 * c + lane;
    const int pc = p < npieces ? p : 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = min((g0 + gl) * R + r, N - 1);
      wq[bf][r] = load_once16(pj.Wp + (int64_t)row * kbytes + 16 * pc);
    }
  };
  const bool has = s0 < s1;
  if (has) {
#pragma unroll
    for (int s = 0; s < P; ++s) fill(s, s0 + s);
  }
  __builtin_amdgcn_sched_barrier(0);

  for (int i = threadIdx.x; i < kStreamMaxRowsWg; i += T) acc_l[i] = 0;
  if (threadIdx.x < 4) reinterpret_cast<i32x4*>(xl + K)[threadIdx.x] = i32x4{0, 0, 0, 0};
  int32_t sx;
  float sc;
  const float gamma = pj.gamma[0];
  if constexpr (KJ > 0) {
    const int K4 = K / 4;
    uint32_t lmax = 0;
#pragma unroll
    for (int j = 0; j < KJ; ++j)
      if (threadIdx.x + T * j < K4) lmax = max(lmax, absmax4(xv[j]));
    lmax = wave_max_u32(lmax);
    if (lane == 0) s_red[0][wave] = lmax;
    __syncthreads();
    uint32_t bmax = s_red[0][0];
#pragma unroll
    for (int w = 1; w < WV; ++w) bmax = max(bmax, s_red[0][w]);
    const float beta = __uint_as_float(bmax);
    const float inv = 127.0f / (beta + 1e-5f);
    const bool write_out = lw == 0 && pj.Xq_out != nullptr;
    int32_t lsum = 0;
#pragma unroll
    for (int j = 0; j < KJ; ++j) {
      const int i = threadIdx.x + T * j;
      if (i < K4) {
        const uint32_t c = quant4(xv[j], inv, lsum);
        reinterpret_cast<uint32_t*>(xl)[i] = c;
        if (write_out) reinterpret_cast<uint32_t*>(pj.Xq_out)[i] = c;
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
      pj.xs_out[0] = sc;
      pj.xsum_out[0] = sx;
    }
  } else {
    sx = pj.xsum[0];
    sc = pj.xs[0];
    __syncthreads();
  }

  int32_t acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0;
  if (has) {
    for (int sb = s0; sb < s1; sb += NB) {
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int s = sb + u;
        if (s < s1) {
          fill((u + P) % NB, s + P);
          const int gl = s / Q, c = s - gl * Q;
          const int p = 64 * c + lane;
          const i32x4* ap = reinterpret_cast<const i32x4*>(xl + (p < npieces ? 64 * p : K));
          int32_t xq[16];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const i32x4 a = ap[v];
            xq[4 * v + 0] = a.x; xq[4 * v + 1] = a.y; xq[4 * v + 2] = a.z; xq[4 * v + 3] = a.w;
          }
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const uint32_t w4[4] = {wq[u][r].x, wq[u][r].y, wq[u][r].z, wq[u][r].w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const i32x4 cd = expand_codes(w4[t]);
              acc[r] = __builtin_amdgcn_sdot4(cd.x, xq[4 * t + 0], acc[r], false);
              acc[r] = __builtin_amdgcn_sdot4(cd.y, xq[4 * t + 1], acc[r], false);
              acc[r] = __builtin_amdgcn_sdot4(cd.z, xq[4 * t + 2], acc[r], false);
              acc[r] = __builtin_amdgcn_sdot4(cd.w, xq[4 * t + 3], acc[r], false);
            }
          }
          if (c == Q - 1 || s == s1 - 1) {
            // the wave leaves this row group: its partial sums into LDS
#pragma unroll
            for (int r = 0; r < R; ++r) {
              const int32_t t = wave_sum_i32(acc[r]);
              if (lane == 0) atomicAdd(&acc_l[gl * R + r], t);
              acc[r] = 0;
            }
          }
        }
      }
    }
  }
  __syncthreads();
  const int rows = (g1 - g0) * R;
  for (int i = threadIdx.x; i < rows; i += T) {
    const int n = g0 * R + i;
    if (n < N) store_out<OUT>(pj.Y, n, acc_l[i] - sx, gamma, sc);
  }
}

// Work shares: workgroups per projection in proportion to its packed bytes
// (each at least one, at most one per row group), at most `nwg` in total; rows
// per workgroup must fit the LDS row accumulators.  Returns the number of
// workgroups to launch, or 0 when the table cannot be served (then another
// kernel takes the call).
inline int stream_plan(StreamArgs& sa, int nwg, int R) {
  double total = 0;
  for (int g = 0; g < sa.G; ++g) total += (double)sa.p[g].N * sa.p[g].K;
  int used = 0;
  for (int g = 0; g < sa.G; ++g) {
    if (sa.p[g].K % 64 != 0 || sa.p[g].K > kStreamMaxK || sa.p[g].N < 1) return 0;
    const int ngroups = (sa.p[g].N + R - 1) / R;
    const int left = nwg - used - (sa.G - 1 - g);   // keep one for each later projection
    int n = (int)((double)nwg * sa.p[g].N * sa.p[g].K / total + 0.5);
    if (g == sa.G - 1) n = left;
    n = std::max(1, std::min(std::min(n, left), ngroups));
    sa.p[g].wg0 = used;
    sa.p[g].nwg = n;
    used += n;
    if ((ngroups + n - 1) / n * R > kStreamMaxRowsWg) return 0;
  }
  for (int g = sa.G; g < kStreamMaxProj; ++g) sa.p[g].wg0 = used;   // never selected
  return used;
}

}  // namespace bl
