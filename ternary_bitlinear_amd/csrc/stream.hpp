// Single-token decode as one persistent launch over one or more projections
// (each with its own fp32 activations, K and N), the quantiser in the
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
//     projections' bytes).  The prologue reaches its first loads after two
//     rounds of argument loads (the projections' first workgroups, then the
//     workgroup's own 32-byte record) and no division: a workgroup's row
//     groups follow from a quotient and remainder computed on the host.
//   - The quantiser (absmax, factor, codes; the same per-element arithmetic
//     as the standalone quantiser) runs once per workgroup into LDS.  The
//     fp32 row's loads go out alone; the first weight loads follow once a
//     wave's part of the row has arrived, and are in flight while the
//     quantiser runs.
//   - The workgroup's work is a list of steps (row group of R rows, chunk of
//     4096 weights); wave w takes a contiguous share of it.  A step loads one
//     16-byte piece of each of the R rows per lane (whole 1 KB lines per
//     wave, with the non-temporal hint: the weights are read once), reads
//     the lane's 64 activations once from LDS for all R rows, and multiplies
//     on the vector ALU (v_dot4_i32_i8 on each 2-bit field of the code bytes
//     masked in place, one accumulator per field: dot_word_fields).
//     Loads run P steps ahead through P + 1 register buffers, so the next
//     loads go out before the current step computes.
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

// What a workgroup needs of its projection before its first loads, in one
// 32-byte record (one scalar load).
struct alignas(32) StreamRec {
  const uint8_t* Wp;
  const float* X;       // fp32 activations [K]
  int N, K;
  int wg0;              // the projection's first workgroup
  // row groups per workgroup: gq, one more for the first gr workgroups
  unsigned short gq, gr;
};

// The launch's table of projections: the first workgroup of each, then their
// records, then what is read only after the dot products.  A workgroup's
// prologue makes two rounds of scalar loads (wg0, then its record).
struct StreamArgs {
  int wg0[kStreamMaxProj];   // first workgroups (wg0[0] = 0); the workgroup count past G
  StreamRec rec[kStreamMaxProj];
  const float* gamma[kStreamMaxProj];
  void* Y[kStreamMaxProj];
  int G;
  // copies of projection 0's quantiser outputs (X~ [K], x_scale, x_sum),
  // written by its first workgroup in the kernel's QOUT form
  int8_t* xq_out;
  float* xs_out;
  int32_t* xsum_out;
};

// The LDS layout of the kernel: activations (K bytes, padded) and a 64-byte
// zero slot, then the row accumulators of the workgroup, then reduction slots.
constexpr int kStreamMaxK = 32768;
constexpr int kStreamMaxRowsWg = 4096;

// QOUT: copy projection 0's quantiser outputs out (xq_out, xs_out, xsum_out).
template <int OUT, int R, int P, int WV, int KJ, bool QOUT>
__global__ __launch_bounds__(WV * kWave) void k_stream(StreamArgs sa) {
  static_assert(KJ > 0, "the fp32 row is held in registers");
  constexpr int NB = P + 1;
  constexpr int T = WV * kWave;
  __shared__ __attribute__((aligned(16))) int8_t xl[kStreamMaxK + 64];
  __shared__ int32_t acc_l[kStreamMaxRowsWg];
  __shared__ uint32_t s_red[2][WV];

  // this workgroup's projection (wg0 past G is the workgroup count, never
  // reached), then its record
  const int b = blockIdx.x;
  int gsel = 0;
#pragma unroll
  for (int i = 1; i < kStreamMaxProj; ++i) gsel += b >= sa.wg0[i] ? 1 : 0;
  const StreamRec rc = sa.rec[gsel];
  const int N = rc.N, K = rc.K;
  const uint8_t* const Wp = rc.Wp;
  const float* const X = rc.X;
  const unsigned lw = (unsigned)(b - rc.wg0);
  const unsigned gq = (unsigned)rc.gq, gr = (unsigned)rc.gr;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const unsigned npieces = (unsigned)K / 64;
  const unsigned Q = (npieces + 63) / 64;             // chunks of 4096 weights per row
  // row groups [g0, g1): gq each, one more for the first gr workgroups
  const int g0 = (int)(lw * gq + min(lw, gr));
  const int g1 = g0 + (int)gq + (lw < gr ? 1 : 0);
  const unsigned S = (unsigned)(g1 - g0) * Q;         // steps of the workgroup
  const int s0 = (int)((unsigned)wave * S / WV);
  const int s1 = (int)((unsigned)(wave + 1) * S / WV);
  const int kbytes = K / 4;

  // the fp32 row first, alone; a thread's loads past K repeat the first
  // value and are not used (loads on every path keep the compiler's waits
  // exact)
  const int K4 = K / 4;
  float4 xv[KJ];
  {
    const float4* src = reinterpret_cast<const float4*>(X);
#pragma unroll
    for (int j = 0; j < KJ; ++j) {
      const int i = threadIdx.x + T * j;
      xv[j] = src[i < K4 ? i : 0];
    }
  }

  uint4 wq[NB][R];
  auto fill = [&](int bf, int s) {
    s = max(min(s, s1 - 1), 0);   // a wave without steps loads step 0 (a valid row)
    const int gl = s / (int)Q, c = s - gl * (int)Q;
    const int p = 64 * c + lane;
    const int pc = p < (int)npieces ? p : 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = min((g0 + gl) * R + r, N - 1);
      wq[bf][r] = load_once16(Wp + (int64_t)row * kbytes + 16 * pc);
    }
  };
  for (int i = threadIdx.x; i < kStreamMaxRowsWg; i += T) acc_l[i] = 0;
  if (threadIdx.x < 4) reinterpret_cast<i32x4*>(xl + K)[threadIdx.x] = i32x4{0, 0, 0, 0};
  uint32_t lmax = 0;
#pragma unroll
  for (int j = 0; j < KJ; ++j)
    if (threadIdx.x + T * j < K4) lmax = max(lmax, absmax4(xv[j]));
  // The first P steps' weight loads go out once this wave's part of the row
  // has arrived, and are in flight while the quantiser runs.  (Issued with
  // the row's loads they compete with them: the row, and so the absmax,
  // arrives later, which costs more than the earlier start gains.)  Every
  // wave issues them, with steps or not, so that the loads are the same on
  // every path and the compiler's waits stay exact.
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s = 0; s < P; ++s) fill(s, s0 + s);
  __builtin_amdgcn_sched_barrier(0);
  lmax = wave_max_u32(lmax);
  if (lane == 0) s_red[0][wave] = lmax;
  __syncthreads();
  uint32_t bmax = s_red[0][0];
#pragma unroll
  for (int w = 1; w < WV; ++w) bmax = max(bmax, s_red[0][w]);
  const float beta = __uint_as_float(bmax);
  const float inv = 127.0f / (beta + 1e-5f);
  int32_t lsum = 0;
#pragma unroll
  for (int j = 0; j < KJ; ++j) {
    const int i = threadIdx.x + T * j;
    if (i < K4) reinterpret_cast<uint32_t*>(xl)[i] = quant4(xv[j], inv, lsum);
  }
  lsum = wave_sum_i32(lsum);
  if (lane == 0) s_red[1][wave] = (uint32_t)lsum;
  __syncthreads();
  int32_t sx = 0;
#pragma unroll
  for (int w = 0; w < WV; ++w) sx += (int32_t)s_red[1][w];
  const float sc = beta / 127.0f;
  if (QOUT && b == 0) {
    // projection 0's first workgroup hands out its quantiser outputs
    for (int i = threadIdx.x; i < K; i += T) sa.xq_out[i] = xl[i];
    if (threadIdx.x == 0) {
      sa.xs_out[0] = sc;
      sa.xsum_out[0] = sx;
    }
  }

  // Per row, one accumulator per 2-bit field of the code bytes
  // (dot_word_fields), added up when the wave leaves the row group.
  int32_t facc[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int f = 0; f < 4; ++f) facc[r][f] = 0;
  // One step: the loads P steps ahead, then the dot products of step s from
  // ring buffer u.
  auto step = [&](const int u, const int s) {
    fill((u + P) % NB, s + P);
    const int gl = s / (int)Q, c = s - gl * (int)Q;
    const int p = 64 * c + lane;
    const i32x4* ap = reinterpret_cast<const i32x4*>(xl + (p < (int)npieces ? 64 * p : K));
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
      for (int t = 0; t < 4; ++t) dot_word_fields(w4[t], &xq[4 * t], facc[r]);
    }
    if (c == (int)Q - 1 || s == s1 - 1) {
      // the wave leaves this row group: its partial sums into LDS
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int32_t t = wave_sum_i32(fields_total(facc[r]));
        if (lane == 0) atomicAdd(&acc_l[gl * R + r], t);
#pragma unroll
        for (int f = 0; f < 4; ++f) facc[r][f] = 0;
      }
    }
  };
  // Whole rounds of NB steps with no guard per step, then the last steps.
  // In a round every load issued for its own steps is also waited for
  // inside it, so at the loop head only the P steps ahead are in flight and
  // the compiler has no reason to drain the ring there.  (With a guard on
  // every step it cannot tell, and waited for every load at the head of
  // each round: 5 % slower on the 7B step.)
  int sb = s0;
  for (; sb + NB <= s1; sb += NB) {
#pragma unroll
    for (int u = 0; u < NB; ++u) step(u, sb + u);
  }
#pragma unroll
  for (int u = 0; u < NB - 1; ++u)
    if (sb + u < s1) step(u, sb + u);
  __syncthreads();
  const float gamma = sa.gamma[gsel][0];
  void* const Y = sa.Y[gsel];
  const int rows = (g1 - g0) * R;
  for (int i = threadIdx.x; i < rows; i += T) {
    const int n = g0 * R + i;
    if (n < N) store_out<OUT>(Y, n, acc_l[i] - sx, gamma, sc);
  }
}

// Work shares: workgroups per projection in proportion to its packed bytes
// (each at least one, at most one per row group), at most `nwg` in total; rows
// per workgroup must fit the LDS row accumulators.  Returns the number of
// workgroups to launch, or 0 when the table cannot be served (then another
// kernel takes the call).
inline int stream_plan(StreamArgs& sa, int nwg, int R) {
  double total = 0;
  for (int g = 0; g < sa.G; ++g) total += (double)sa.rec[g].N * sa.rec[g].K;
  int used = 0;
  for (int g = 0; g < sa.G; ++g) {
    if (sa.rec[g].K % 64 != 0 || sa.rec[g].K > kStreamMaxK || sa.rec[g].N < 1) return 0;
    const int ngroups = (sa.rec[g].N + R - 1) / R;
    const int left = nwg - used - (sa.G - 1 - g);   // keep one for each later projection
    int n = (int)((double)nwg * sa.rec[g].N * sa.rec[g].K / total + 0.5);
    if (g == sa.G - 1) n = left;
    n = std::max(1, std::min(std::min(n, left), ngroups));
    sa.wg0[g] = used;
    sa.rec[g].wg0 = used;
    sa.rec[g].gq = (unsigned short)(ngroups / n);
    sa.rec[g].gr = (unsigned short)(ngroups % n);
    used += n;
    if ((ngroups + n - 1) / n * R > kStreamMaxRowsWg) return 0;
  }
  for (int g = sa.G; g < kStreamMaxProj; ++g) sa.wg0[g] = used;   // never selected
  return used;
}

}  // namespace bl
