// Calibration kernels (measurement aids, not part of the method): MFMA
// throughput with the shader clock, and the streaming-read rate of HBM.
//
// MFMA throughput and shader-clock calibration.  Each wavefront issues
// v_mfma_f32_32x32x16_bf16 back to back on four independent accumulators, its
// A and B operands cycling through eight register sets so that consecutive
// products see different data; the workgroup records the shader-clock cycles
// (s_memtime) and the 100 MHz constant-clock ticks (s_memrealtime) it spent.
#include "device_common.hpp"
#include "kernels.h"

namespace tpmlp {
namespace {

constexpr int CAL_THREADS = 256;  // 4 wavefronts: one per SIMD

// A pseudo-normal bf16 from a hash (sum of four uniforms, scaled).
__device__ __forceinline__ bf16 hashed_normal(uint32_t h, float scale) {
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    h ^= h >> 13;
    h *= 0x5bd1e995u;
    h ^= h >> 15;
    s += (float)(h & 0xffff) * (1.0f / 65536.0f);
  }
  return (bf16)((s - 2.0f) * 1.7320508f * scale);
}

__global__ __launch_bounds__(CAL_THREADS) void calib_mfma_kernel(int gaussian, int64_t iters,
                                                                 uint64_t *stats) {
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  bf16x8 a[8], b[8];
  const uint32_t seed = (blockIdx.x * CAL_THREADS + threadIdx.x) * 2654435761u;
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[r][e] = gaussian ? hashed_normal(seed ^ (r * 8 + e) * 0x9e3779b9u, 1.0f) : (bf16)0.0f;
      b[r][e] = gaussian ? hashed_normal(seed ^ (64 + r * 8 + e) * 0x85ebca6bu, 0.02f) : (bf16)0.0f;
    }
  f32x16 acc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[q][v] = 0.0f;
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[(3 * j + 1) & 7], acc[j & 3], 0,
                                                           0, 0);
  }
  // Keep the products live: one value per lane (sum of the accumulators).
  float s = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[q][v];
  __syncthreads();
  if (threadIdx.x == 0) {
    stats[2 * blockIdx.x] = __builtin_amdgcn_s_memtime() - c0;
    stats[2 * blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime() - r0;
  }
  // A data-dependent store that never happens for finite sums keeps the
  // compiler from dropping the loop.
  if (s != s) stats[2 * blockIdx.x] = 0;
}

// Streaming read of `n16` 16-byte chunks: workgroup b reads the contiguous
// range [b c, (b+1) c), c = ceil(n16 / nwg), its 256 threads on consecutive
// 16-byte chunks, 8 loads in flight per thread, with the nontemporal hint (as
// the few-token kernels read weights).  The loads are folded into one word,
// stored only when it equals one particular value, so they cannot be dropped
// and (almost) nothing is written.  Of the patterns measured (a grid-stride
// walk over the whole buffer, this per-workgroup range, 2 to 16 loads in
// flight, 256 to 8192 workgroups, with and without the hint) this one read
// fastest.
constexpr int HBM_THREADS = 256;
constexpr int HBM_UNROLL = 8;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(HBM_THREADS) void calib_hbm_read_kernel(const u32x4 *p, int64_t n16,
                                                                     uint32_t *sink) {
  const int64_t c = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t beg = (int64_t)blockIdx.x * c;
  const int64_t end = beg + c < n16 ? beg + c : n16;
  uint32_t acc = 0;
  int64_t i = beg + threadIdx.x;
  for (; i + (HBM_UNROLL - 1) * HBM_THREADS < end; i += HBM_UNROLL * HBM_THREADS) {
    u32x4 v[HBM_UNROLL];
#pragma unroll
    for (int j = 0; j < HBM_UNROLL; ++j) v[j] = __builtin_nontemporal_load(p + i + j * HBM_THREADS);
#pragma unroll
    for (int j = 0; j < HBM_UNROLL; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
  }
  for (; i < end; i += HBM_THREADS) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

}  // namespace

hipError_t launch_calib_hbm_read(const void *buf, int64_t bytes, uint32_t *sink, int nwg,
                                 hipStream_t s) {
  hipLaunchKernelGGL(calib_hbm_read_kernel, dim3((unsigned)nwg), dim3(HBM_THREADS), 0, s,
                     (const u32x4 *)buf, bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_calib_mfma(int gaussian, int64_t iters, uint64_t *stats, int nwg, hipStream_t s) {
  hipLaunchKernelGGL(calib_mfma_kernel, dim3((unsigned)nwg), dim3(CAL_THREADS), 0, s, gaussian,
                     iters, stats);
  return hipGetLastError();
}

}  // namespace tpmlp
