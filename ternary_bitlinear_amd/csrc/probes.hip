// Chip-limit probes for the bench (not part of the BitLinear ABI; built into
// libbitlinear_probes.so and loaded only by bench.py): a plain streaming read
// of a buffer (plain loads or with the non-temporal hint), the floor any
// kernel that must read the same bytes can reach;
// a read of one buffer by every workgroup, the rate at which a CU takes in
// data all CUs share (the skinny kernels' activations); and a loop of int8
// matrix instructions on register operands with the value
// distributions of the projection (codes in {0, 1, 2}, quantised activations)
// in either operand order, the ceiling of the matrix cores for those operands.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));

// Grid-stride read of n16 16-byte pieces, UNROLL loads in flight per thread,
// plain or with the non-temporal hint (NT); the XOR of everything read is
// stored only if it equals an unlikely value, so the loads cannot be removed
// and nothing is written.
template <int UNROLL, bool NT>
__global__ __launch_bounds__(256) void k_stream_read(const uint4* __restrict__ p, int64_t n16,
                                                     uint32_t* __restrict__ sink) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  uint32_t a = 0;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (; i + (UNROLL - 1) * stride < n16; i += UNROLL * stride) {
    uint4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      if constexpr (NT) {
        const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + i + u * stride));
        v[u] = make_uint4(t.x, t.y, t.z, t.w);
      } else {
        v[u] = p[i + u * stride];
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) a ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = p[i];
    a ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (a == 0x9e3779b9u) sink[0] = a;
}

// Every workgroup reads the whole buffer (n16 16-byte pieces, UNROLL loads in
// flight per thread): with one workgroup per CU and a buffer that L2 holds,
// the rate at which one CU can take in data that all CUs share.
template <int UNROLL>
__global__ __launch_bounds__(512) void k_bcast_read(const uint4* __restrict__ p, int64_t n16,
                                                    uint32_t* __restrict__ sink) {
  uint32_t a = 0;
  int64_t i = threadIdx.x;
  for (; i + (UNROLL - 1) * 512 < n16; i += UNROLL * 512) {
    uint4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) v[u] = p[i + u * 512];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) a ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += 512) {
    const uint4 v = p[i];
    a ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (a == 0x9e3779b9u) sink[0] = a;
}

// iters x 16 independent v_mfma_i32_32x32x32_i8 per wave (4 accumulator
// sets), operands from registers.  mode 1: the first operand holds codes in
// {0, 1, 2} and the second int8 values spread like quantised activations (a
// triangular spread, |x| < 64); mode 2: the same values with the operands
// exchanged (activations first, the GEMM's order); mode 0: both zero.  The
// matrix cores draw less power on constant operands, and less with the
// codes second than first.  The accumulators are stored only if their sum
// equals an unlikely value.
__global__ __launch_bounds__(256) void k_mfma_loop(int iters, int mode, int32_t* __restrict__ sink) {
  const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t h = (blockIdx.x * 4 + wave) * 64 + lane;
  auto next = [&]() {
    h ^= h << 13; h ^= h >> 17; h ^= h << 5;
    return h;
  };
  i32x4 a[4], b[4];
  for (int s = 0; s < 4; ++s) {
    for (int d = 0; d < 4; ++d) {
      uint32_t ca = 0, xb = 0;
      for (int byte = 0; byte < 4; ++byte) {
        uint32_t r = next();
        ca |= (r % 3u) << (8 * byte);
        // a sum of two small uniforms: a triangular spread around 0
        const int x = (int)((r >> 8) & 63u) - (int)((r >> 16) & 63u);
        xb |= ((uint32_t)x & 0xffu) << (8 * byte);
      }
      a[s][d] = mode == 1 ? (int32_t)ca : mode == 2 ? (int32_t)xb : 0;
      b[s][d] = mode == 1 ? (int32_t)xb : mode == 2 ? (int32_t)ca : 0;
    }
  }
  i32x16 acc[4];
  for (int s = 0; s < 4; ++s)
    for (int e = 0; e < 16; ++e) acc[s][e] = 0;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc[s] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[(s + r) & 3], b[s], acc[s], 0, 0, 0);
  }
  int32_t t = 0;
  for (int s = 0; s < 4; ++s)
    for (int e = 0; e < 16; ++e) t += acc[s][e];
  if (t == 0x7eadbeef) sink[0] = t;
}

}  // namespace

extern "C" {

// Plain read of `bytes` (a multiple of 16, 16-byte aligned) at `p` with
// `grid` workgroups of 256 threads; nt != 0: loads with the non-temporal
// hint.  Returns a hipError_t.
int probe_stream_read(const void* p, size_t bytes, int grid, int nt, void* sink, void* stream) {
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint4* q = reinterpret_cast<const uint4*>(p);
  uint32_t* s = reinterpret_cast<uint32_t*>(sink);
  if (nt)
    k_stream_read<4, true><<<dim3(grid), dim3(256), 0, st>>>(q, (int64_t)(bytes / 16), s);
  else
    k_stream_read<4, false><<<dim3(grid), dim3(256), 0, st>>>(q, (int64_t)(bytes / 16), s);
  return (int)hipGetLastError();
}

// Shared read: `grid` workgroups of 512 threads each read all `bytes` (a
// multiple of 16, 16-byte aligned) at `p`.  Returns a hipError_t.
int probe_bcast_read(const void* p, size_t bytes, int grid, void* sink, void* stream) {
  k_bcast_read<4><<<dim3(grid), dim3(512), 0, reinterpret_cast<hipStream_t>(stream)>>>(
      reinterpret_cast<const uint4*>(p), (int64_t)(bytes / 16), reinterpret_cast<uint32_t*>(sink));
  return (int)hipGetLastError();
}

// int8 matrix-instruction loop: grid x 4 waves x iters x 16 instructions of
// 2 * 32 * 32 * 32 operations each, on the projection's operand values (mode
// 1: codes first; mode 2: activations first) or on zeros (mode 0).  Returns
// a hipError_t.
int probe_mfma_loop(int iters, int mode, int grid, void* sink, void* stream) {
  k_mfma_loop<<<dim3(grid), dim3(256), 0, reinterpret_cast<hipStream_t>(stream)>>>(
      iters, mode, reinterpret_cast<int32_t*>(sink));
  return (int)hipGetLastError();
}

}  // extern "C"
