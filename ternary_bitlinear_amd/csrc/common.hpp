// Device helpers shared by the BitLinear kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

constexpr int kWave = 64;

// ---- integer / bit helpers --------------------------------------------------
__device__ __forceinline__ uint32_t abs_bits(float x) { return __float_as_uint(x) & 0x7fffffffu; }

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---- activation quantiser ----------------------------------------------------
// x~ = RoundClip(x * inv, -127, 127) with inv = 127 / (beta + eps) already in
// fp32: one fp32 multiply, then floor(q + 1/2) taken exactly as
// floor(q) + (q - floor(q) >= 1/2) (q - floor(q) is exact for |q| < 2^23).
// Sources are built without contraction, so the multiply never fuses with the
// subtraction.
__device__ __forceinline__ int32_t quant1(float x, float inv) {
  const float q = x * inv;
  const float r = floorf(q);
  int32_t v = (int32_t)r + ((q - r) >= 0.5f ? 1 : 0);
  return max(-127, min(127, v));
}

// Four values -> four int8 codes packed little endian; adds them to `sum`.
__device__ __forceinline__ uint32_t quant4(const float4& f, float inv, int32_t& sum) {
  const int32_t a = quant1(f.x, inv), b = quant1(f.y, inv), c = quant1(f.z, inv),
                d = quant1(f.w, inv);
  sum += a + b + c + d;
  return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
         ((uint32_t)(d & 0xff) << 24);
}

__device__ __forceinline__ uint32_t absmax4(const float4& f) {
  return max(max(abs_bits(f.x), abs_bits(f.y)), max(abs_bits(f.z), abs_bits(f.w)));
}

// ---- wave reductions (all 64 lanes active; every lane receives the result) --
// In the vector ALU with DPP, no round trip through the LDS crossbar: an
// inclusive prefix within each row of 16 lanes (row_shr 1, 2, 4, 8), then the
// last lane of a row carried into the next rows (row_bcast15 into rows 1 and
// 3, row_bcast31 into rows 2 and 3), so lane 63 ends with the whole wave's
// value and readlane makes it uniform.  Lanes shifted in from outside a row,
// and rows outside a step's row mask, contribute 0: the identity of both
// wrapping addition and unsigned max.
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, Op op) {
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true));   // row_shr:1
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true));   // row_shr:2
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true));   // row_shr:4
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true));   // row_shr:8
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, true));   // row_bcast15
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, true));   // row_bcast31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return wave_reduce_u32(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}

__device__ __forceinline__ int32_t wave_sum_i32(int32_t v) {
  return (int32_t)wave_reduce_u32((uint32_t)v, [](uint32_t a, uint32_t b) { return a + b; });
}

// 64-bit sum over the wave by the same DPP steps, each moving both 32-bit
// halves of a value; every lane receives the result.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, ROW_MASK, 0xF, true);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, ROW_MASK, 0xF, true);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_sum_u64_dpp(uint64_t v) {
  v += dpp_u64<0x111, 0xF>(v);   // row_shr:1
  v += dpp_u64<0x112, 0xF>(v);   // row_shr:2
  v += dpp_u64<0x114, 0xF>(v);   // row_shr:4
  v += dpp_u64<0x118, 0xF>(v);   // row_shr:8
  v += dpp_u64<0x142, 0xA>(v);   // row_bcast15
  v += dpp_u64<0x143, 0xC>(v);   // row_bcast31
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// fp64 sum over the wave by the same DPP steps; every lane receives the
// result.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_f64(double v) {
  return __longlong_as_double((long long)dpp_u64<CTRL, ROW_MASK>((uint64_t)__double_as_longlong(v)));
}

__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64<0x111, 0xF>(v);   // row_shr:1
  v += dpp_f64<0x112, 0xF>(v);   // row_shr:2
  v += dpp_f64<0x114, 0xF>(v);   // row_shr:4
  v += dpp_f64<0x118, 0xF>(v);   // row_shr:8
  v += dpp_f64<0x142, 0xA>(v);   // row_bcast15
  v += dpp_f64<0x143, 0xC>(v);   // row_bcast31
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), 63);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// ---- exact mean of squares (RMS normalisation) ------------------------------
// RMS normalisation of a token (page section 2: the activations are
// RMS-normalised before the quantiser; the normalisation of the reference it
// cites): y_k = x_k / sqrt(mean_k x_k^2 + eps) * g_k.  The mean of squares is
// the exact rational sum_k x_k^2 / K rounded once to fp32 (nearest, ties to
// even), so it does not depend on how a launch splits the row.
//
// An fp32 x is sig 2^(eb - 150) with eb = max(exponent field, 1) and sig its
// 24-bit significand, so x^2 = sig^2 2^(2 eb - 300), sig^2 < 2^48.  Against an
// anchor exponent lb, a value with lb <= eb <= lb + kSqWindow adds
// sig^2 << 2 (eb - lb) (< 2^110) in units of 2^(2 lb - 300); at most 2^17 such
// values (K <= 131072) sum below 2^127, so an unsigned 128-bit integer holds
// the sum exactly.  The first window is anchored 31 exponents below the row's
// largest; values further down (more than 2^31 times smaller than the row's
// largest magnitude, so rare) are summed in further windows, each 32
// exponents lower, added into a multi-word integer.
typedef unsigned __int128 u128;
constexpr int kSqWindow = 31;
constexpr int kSqLimbs = 18;   // 32-bit words of sum x^2 in units of 2^-298 (top bit < 572)

__device__ __forceinline__ int sq_eb(uint32_t bits) { return max((int)(bits >> 23), 1); }

// acc += x^2 in units of 2^(2 lb - 300) when lb <= eb(x) <= hi (hi - lb <=
// kSqWindow); returns true when x is non-zero and below the window.
struct SqAcc {
  uint64_t lo = 0, hi = 0;
};
__device__ __forceinline__ bool sq_add(SqAcc& a, float x, int lb, int hi) {
  const uint32_t b = abs_bits(x);
  const int eb = sq_eb(b);
  const uint32_t sig = (b & 0x7fffffu) | ((b >> 23) ? 0x800000u : 0u);
  const uint64_t q = (uint64_t)sig * sig;
  const bool in = eb >= lb && eb <= hi;
  const uint32_t sh = in ? 2u * (uint32_t)(eb - lb) : 0u;   // 0 .. 62
  const uint64_t lo = in ? q << sh : 0ull;
  const uint64_t up = in ? (q >> 1) >> (63u - sh) : 0ull;   // q >> (64 - sh), 0 for sh = 0
  a.lo += lo;
  a.hi += up + (a.lo < lo ? 1ull : 0ull);
  return eb < lb && q != 0;
}

// Sum over the wave of 128-bit values whose total is below 2^128: each
// 32-bit limb is summed as a 64-bit value (64 lanes x 2^32 < 2^38), then the
// limb sums are recombined.
__device__ __forceinline__ u128 wave_sum_u128(const SqAcc& a) {
  const uint64_t l0 = wave_sum_u64_dpp(a.lo & 0xffffffffull);
  const uint64_t l1 = wave_sum_u64_dpp(a.lo >> 32);
  const uint64_t l2 = wave_sum_u64_dpp(a.hi & 0xffffffffull);
  const uint64_t l3 = wave_sum_u64_dpp(a.hi >> 32);
  return (u128)l0 + ((u128)l1 << 32) + ((u128)l2 << 64) + ((u128)l3 << 96);
}

// RN32((T + f) 2^e2 / K) for T in [2^63, 2^64), 0 <= f < 1 (f > 0 exactly when
// `sticky`), 1 <= K <= 2^17: the quotient q = floor(T / K) has at least 47
// bits, and (T + f) / K = q + (r + f) / K with 0 <= (r + f) / K < 1, zero only
// when the remainder r and f both are.  Nearest, ties to even; subnormal
// results and overflow to infinity as fp32 rounding has them.
__device__ __forceinline__ float rn32_quotient(uint64_t T, bool sticky, int e2, uint32_t K) {
  const uint64_t q = T / (uint64_t)K;
  const bool st = sticky || q * (uint64_t)K != T;
  const int pq = 63 - __clzll((long long)q);
  const int lsb = max(pq - 23, -149 - e2);   // >= 23
  if (lsb > 64) return 0.f;                  // below 2^-150
  const uint64_t sig0 = lsb >= 64 ? 0ull : q >> lsb;
  const uint32_t guard = (uint32_t)((q >> (lsb - 1)) & 1ull);
  const bool rest = st || (q & ((1ull << (lsb - 1)) - 1ull)) != 0;
  uint64_t sig = sig0 + ((guard && (rest || (sig0 & 1ull))) ? 1ull : 0ull);
  int ex = lsb + e2;                         // value = sig 2^ex
  if (sig == (1ull << 24)) { sig >>= 1; ++ex; }
  if (sig == 0) return 0.f;
  if (ex + 23 > 127) return __uint_as_float(0x7f800000u);
  if (sig < (1ull << 23)) return __uint_as_float((uint32_t)sig);   // subnormal (ex = -149)
  return __uint_as_float(((uint32_t)(ex + 150) << 23) | ((uint32_t)sig & 0x7fffffu));
}

// RN32(V 2^ue / K) for a 128-bit V.
__device__ __forceinline__ float mean_sq_u128(u128 V, int ue, uint32_t K) {
  if (V == 0) return 0.f;
  const uint64_t h = (uint64_t)(V >> 64), l = (uint64_t)V;
  const int p = h ? 127 - __clzll((long long)h) : 63 - __clzll((long long)l);
  if (p < 63) return rn32_quotient(l << (63 - p), false, ue + p - 63, K);
  const int d = p - 63;                      // 0 .. 64
  const uint64_t T = (uint64_t)(V >> d);
  const bool st = d > 0 && (V & ((((u128)1) << d) - 1)) != 0;
  return rn32_quotient(T, st, ue + d, K);
}

// big += v << off (off even, v < 2^127; the total stays below 2^576).
__device__ inline void big_add(uint32_t* big, u128 v, int off) {
  const int i0 = off >> 5, sh = off & 31;
  const u128 lowp = v << sh;
  const uint32_t w0 = (uint32_t)lowp, w1 = (uint32_t)(lowp >> 32), w2 = (uint32_t)(lowp >> 64),
                 w3 = (uint32_t)(lowp >> 96), w4 = sh ? (uint32_t)(v >> (128 - sh)) : 0u;
  uint64_t carry = 0;
#pragma unroll 1
  for (int i = i0; i < kSqLimbs; ++i) {
    const int d = i - i0;
    const uint32_t add = d == 0 ? w0 : d == 1 ? w1 : d == 2 ? w2 : d == 3 ? w3 : d == 4 ? w4 : 0u;
    const uint64_t t = (uint64_t)big[i] + add + carry;
    big[i] = (uint32_t)t;
    carry = t >> 32;
    if (d >= 4 && carry == 0) break;
  }
}

// RN32(big 2^-298 / K).
__device__ inline float mean_sq_big(const uint32_t* big, uint32_t K) {
  int t = kSqLimbs - 1;
  while (t >= 0 && big[t] == 0) --t;
  if (t < 0) return 0.f;
  const int p = 32 * t + 31 - __clz(big[t]);
  auto bit = [&](int b) -> uint64_t { return (big[b >> 5] >> (b & 31)) & 1u; };
  if (p < 63) {
    uint64_t v = 0;
    for (int b = p; b >= 0; --b) v = (v << 1) | bit(b);
    return rn32_quotient(v << (63 - p), false, p - 63 - 298, K);
  }
  uint64_t T = 0;
  for (int b = p; b >= p - 63; --b) T = (T << 1) | bit(b);
  bool st = false;
  for (int b = p - 64; b >= 0 && !st; --b) st = bit(b) != 0;
  return rn32_quotient(T, st, p - 63 - 298, K);
}

// Workgroup scratch of block_mean_square (T threads).
template <int T>
struct SqShared {
  double wsq[T / kWave];
  uint32_t wmax[T / kWave];
  uint64_t wsum[T / kWave][2];
  uint32_t wtail[T / kWave];
  uint32_t big[kSqLimbs];
  float ms;
};

// One window [lb, hi] of the row: every thread receives the exact 128-bit sum
// and whether any value lies below lb.  Thread t reads the float4 groups t,
// t + T, ... of the row (the partition does not matter: the sum is exact).
// `again`: the scratch was read by a previous window (wait for those reads
// first).
template <int T>
__device__ __forceinline__ u128 block_sq_window(const float4* row, int64_t K4, int lb, int hi,
                                                SqShared<T>& sh, bool again, bool& tail) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  SqAcc a;
  bool tl = false;
#pragma unroll 1
  for (int64_t i = threadIdx.x; i < K4; i += T) {
    const float4 x = row[i];
    tl |= sq_add(a, x.x, lb, hi);
    tl |= sq_add(a, x.y, lb, hi);
    tl |= sq_add(a, x.z, lb, hi);
    tl |= sq_add(a, x.w, lb, hi);
  }
  const u128 w = wave_sum_u128(a);
  const bool wt = __any(tl);
  if (again) __syncthreads();
  if (lane == 0) {
    sh.wsum[wave][0] = (uint64_t)w;
    sh.wsum[wave][1] = (uint64_t)(w >> 64);
    sh.wtail[wave] = wt ? 1u : 0u;
  }
  __syncthreads();
  u128 v = 0;
  uint32_t t = 0;
#pragma unroll 1
  for (int i = 0; i < T / kWave; ++i) {
    v += ((u128)sh.wsum[i][1] << 64) | sh.wsum[i][0];
    t |= sh.wtail[i];
  }
  tail = t != 0;
  return v;
}

// The exact sum in integer windows (see above), rounded once; the row is read
// again from memory.
template <int T>
__device__ float block_mean_square_exact(const float4* row, int64_t K4, uint32_t K,
                                         SqShared<T>& sh) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  uint32_t mx = 0;
#pragma unroll 1
  for (int64_t i = threadIdx.x; i < K4; i += T) {
    const float4 x = row[i];
    mx = max(mx, absmax4(x));
  }
  mx = wave_max_u32(mx);
  if (lane == 0) sh.wmax[wave] = mx;
  __syncthreads();
#pragma unroll 1
  for (int i = 0; i < T / kWave; ++i) mx = max(mx, sh.wmax[i]);
  int hi = sq_eb(mx);
  int lb = max(hi - kSqWindow, 1);
  bool tail;
  u128 v = block_sq_window<T>(row, K4, lb, hi, sh, false, tail);
  if (!tail) return mean_sq_u128(v, 2 * lb - 300, K);
  // Values below the first window: further windows, added exactly into a
  // multi-word integer (units of 2^-298) by thread 0.
  if (threadIdx.x == 0) {
    for (int i = 0; i < kSqLimbs; ++i) sh.big[i] = 0;
    big_add(sh.big, v, 2 * lb - 2);
  }
  while (tail) {   // uniform; ends by lb = 1 at the latest
    hi = lb - 1;
    lb = max(hi - kSqWindow, 1);
    v = block_sq_window<T>(row, K4, lb, hi, sh, true, tail);
    if (threadIdx.x == 0) big_add(sh.big, v, 2 * lb - 2);
  }
  if (threadIdx.x == 0) sh.ms = mean_sq_big(sh.big, K);
  __syncthreads();
  return sh.ms;
}

// RN32(sum x^2 / K) over one row whose values the T threads of the
// workgroup hold: visit(f) calls f(x) on each group of four values this
// thread holds (zero padding allowed).  Every thread of the workgroup must call it; all receive
// the same value and the same return flag.  Returns false when the fp64 sum
// cannot decide the rounding: the caller then takes block_mean_square_exact
// (which reads the row again from memory, so a caller that holds the row in
// registers reloads it afterwards and keeps nothing live across that path).
//
// The fp64 sum: every square is exact in fp64 (48-bit significand, exponent
// within range) and every term is non-negative, so any summation order errs
// by at most (n - 1) 2^-53 (1 + O(n 2^-53)) of the exact sum S, and the fp64
// quotient by K adds one more rounding.  With e = 4 K 2^-53 (at least twice
// that bound for K >= 16), the exact mean lies in [m - e m, m + e m] around
// the fp64 mean m; rounding is monotone, so when both ends round to the same
// fp32 value, so does the exact mean.  Otherwise (the exact mean within about
// K 2^-51 of a rounding boundary: a few rows in 2^(29 - log2 K), and every
// exact tie) the exact integer sum decides.
template <int T, typename Visit>
__device__ __forceinline__ bool block_mean_square_fast(Visit visit, uint32_t K, SqShared<T>& sh,
                                                       float& ms) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  double s = 0.0;
  visit([&](const float4& x) {
    const double a = x.x, b = x.y, c = x.z, d = x.w;
    s += ((a * a + b * b) + c * c) + d * d;
  });
  s = wave_sum_f64(s);
  if (lane == 0) sh.wsq[wave] = s;
  __syncthreads();
  double tot = 0.0;
#pragma unroll
  for (int i = 0; i < T / kWave; ++i) tot += sh.wsq[i];
  const double m = tot / (double)K;
  const double e = m * ((double)(4 * K) * 0x1p-53);
  const float lo = (float)(m - e), hi = (float)(m + e);
  ms = lo;
  return lo == hi;
}

// r = 1 / sqrt(ms + eps) from the fp32 mean of squares: an fp32 add, then a
// correctly rounded fp32 square root and reciprocal; each element is then
// fl32(fl32(x_k r) g_k) (rms_apply).
__device__ __forceinline__ float rms_reciprocal(float ms) {
  return 1.0f / sqrtf(ms + 1e-5f);
}

__device__ __forceinline__ float4 rms_apply(const float4& x, float r, const float4& g) {
  return make_float4((x.x * r) * g.x, (x.y * r) * g.y, (x.z * r) * g.z, (x.w * r) * g.w);
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += (uint64_t)__shfl_xor((unsigned long long)v, o, kWave);
  return v;
}

// ---- output store (page section 2 rescale; section 6 "Scaling Factor Fusion") --
constexpr int kOutF32 = 0, kOutBF16 = 1, kOutI32 = 2;

// y = fl32(fl32((float)acc * gamma) * scale), stored as fp32 or bf16 (nearest
// even); int32 output stores acc itself.
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

// ---- MFMA int8 operand types --------------------------------------------------
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// 16 bytes that the kernel reads exactly once (packed weights), loaded with
// the non-temporal hint.  Timed on MI355X: a streaming read with the hint
// runs 4-7 % faster than with plain loads; the multi-projection and
// vector-ALU single-token kernels 6 % faster, the skinny kernel 0-4 % (its
// direct-to-LDS code loads).  Not every access pattern gains: the matrix
// decode kernel lost 7-11 % with it and keeps plain loads.
__device__ __forceinline__ uint4 load_once16(const void* p) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}
// The same hint as the cache-policy argument of a direct global->LDS load.
constexpr int kLdsLoadOnce = 2;

// v_mfma_i32_16x16x64_i8: C[16x16] += A[16x64] * B[64x16].
// Lane l supplies A row (l % 16) and B column (l % 16) for k-group (l / 16);
// the 16 bytes of a lane's A and B operands pair up byte for byte, so any
// assignment of k values to (k-group, byte) slots works as long as A and B use
// the same one.  Result: lane l, register r holds C[4 * (l / 16) + r][l % 16].
__device__ __forceinline__ i32x4 mfma_i8_16x16x64(i32x4 a, i32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

typedef int32_t i32x16 __attribute__((ext_vector_type(16)));

// v_mfma_i32_32x32x32_i8: C[32x32] += A[32x32] * B[32x32].  Lane l supplies A
// row (l % 32) and B column (l % 32) for k-group (l / 32), 16 bytes each,
// paired byte for byte as in the 16x16 form.  Result: lane l, register r
// holds C[8 * (r / 4) + 4 * (l / 32) + (r % 4)][l % 32].
__device__ __forceinline__ i32x16 mfma_i8_32x32x32(i32x4 a, i32x4 b, i32x16 c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// Four int8 codes per dword from one packed BLT2 word: dword d holds the codes
// (W~ + 1, values 0..2) of k = 16g + 4d .. 16g + 4d + 3, i.e. the 16 codes of
// the word in natural k order.
__device__ __forceinline__ i32x4 expand_codes(uint32_t w) {
  i32x4 r;
  r.x = (int32_t)(w & 0x03030303u);
  r.y = (int32_t)((w >> 2) & 0x03030303u);
  r.z = (int32_t)((w >> 4) & 0x03030303u);
  r.w = (int32_t)((w >> 6) & 0x03030303u);
  return r;
}

// sum_k c_k x~_k of one 16-code word w (BLT2-v1) against its 16 activations,
// four per dword in k order (x[d] holds k = 4d .. 4d + 3), on the vector ALU
// without expanding the codes to bytes: field f of the code bytes (bits 2f,
// 2f + 1 of byte b: the code of k = 4f + b) is masked in place, so its bytes
// are c 4^f for f = 0, 1, 2, and field 3 is shifted down one bit (c 32, at
// most 64, still a signed byte).  One accumulator per field; fields_total
// divides each back exactly (every field sum is a multiple of its scale).
// Five masks and four v_dot4 per word, against seven and four for the byte
// expansion.  An accumulator stays below 2^31 while |sum| <= 2 * 127 * 32 K,
// i.e. for any K below 2^18.
__device__ __forceinline__ void dot_word_fields(uint32_t w, const int32_t* x, int32_t (&acc)[4]) {
  acc[0] = __builtin_amdgcn_sdot4((int32_t)(w & 0x03030303u), x[0], acc[0], false);
  acc[1] = __builtin_amdgcn_sdot4((int32_t)(w & 0x0c0c0c0cu), x[1], acc[1], false);
  acc[2] = __builtin_amdgcn_sdot4((int32_t)(w & 0x30303030u), x[2], acc[2], false);
  acc[3] = __builtin_amdgcn_sdot4((int32_t)((w >> 1) & 0x60606060u), x[3], acc[3], false);
}

__device__ __forceinline__ int32_t fields_total(const int32_t (&acc)[4]) {
  return acc[0] + (acc[1] >> 2) + (acc[2] >> 4) + (acc[3] >> 5);
}

}  // namespace bl
