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

// fp64 sum over the wave by the same DPP steps, each moving both 32-bit halves
// of a value; every lane receives the result.  The addition order is fixed,
// so the result is reproducible.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, ROW_MASK, 0xF, true);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, ROW_MASK, 0xF, true);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
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

// RMS normalisation of a token (page section 2: activations are RMS-normalised
// before the quantiser; the normalisation of the reference it cites):
// y_k = x_k / sqrt(mean x^2 + eps) * g_k.  sq is the token's sum of squares in
// fp64 (each square exact); ms = fl32(sq / K), then an fp32 add, a correctly
// rounded fp32 square root and reciprocal.  Returns r; each element is then
// fl32(fl32(x_k r) g_k) (rms_apply).
__device__ __forceinline__ float rms_reciprocal(double sq, int64_t K) {
  const float ms = (float)(sq / (double)K);
  return 1.0f / sqrtf(ms + 1e-5f);
}

__device__ __forceinline__ float4 rms_apply(const float4& x, float r, const float4& g) {
  return make_float4((x.x * r) * g.x, (x.y * r) * g.y, (x.z * r) * g.z, (x.w * r) * g.w);
}

__device__ __forceinline__ double sum_sq4(const float4& x) {
  const double a = x.x, b = x.y, c = x.z, d = x.w;
  return ((a * a + b * b) + c * c) + d * d;
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

}  // namespace bl
