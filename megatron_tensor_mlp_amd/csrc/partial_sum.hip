// The reduction of p fp32 partials on one device: what the all-reduce of the
// row-parallel step computes (Day 41 post, "Simulating row parallel linear":
// the partials are summed, then the row bias is added once).
//
// HBM-bound: every element of every partial is read once and Z is written
// once.  Each thread owns 16-byte (4-float) chunks, reads all p partials of a
// chunk before adding (the loads are independent, so they are all in flight
// together), and adds them shard 0 first, then b2, so the result equals a
// left-to-right fp32 sum bit for bit.  Every byte is touched once, so loads
// and stores are nontemporal (they do not displace cached data; measured
// 5.4 -> 6.2 TB/s on the 8 x [512, 8192] reduction).  A grid-stride loop keeps
// the launch a fixed multiple of the CU count.
#include "device_common.hpp"
#include "kernels.h"

namespace tpmlp {
namespace {

constexpr int THREADS = 256;

__global__ __launch_bounds__(THREADS) void partial_sum_kernel(const PartSumArgs a) {
  const int64_t d4 = a.d / 4;
  const int64_t total = a.T * d4;
  const int64_t stride = (int64_t)gridDim.x * THREADS;
  for (int64_t c = (int64_t)blockIdx.x * THREADS + threadIdx.x; c < total; c += stride) {
    const int64_t t = c / d4, c4 = c - t * d4;
    const int64_t off = t * a.ldp + 4 * c4;
    // Partials in groups of 8: all loads of a group are issued first (shards
    // past p re-read the last one and are not added), then added in order.
    f32x4 acc;
    for (int q = 0; q < a.p; q += 8) {
      f32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = __builtin_nontemporal_load(
            (const f32x4 *)(a.parts[q + u < a.p ? q + u : a.p - 1] + off));
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (q + u >= a.p) break;
        acc = (q + u == 0) ? v[u] : acc + v[u];
      }
    }
    if (a.b2) acc += *(const f32x4 *)(a.b2 + 4 * c4);
    __builtin_nontemporal_store(acc, (f32x4 *)(a.Z + t * a.ldz + 4 * c4));
  }
}

}  // namespace

hipError_t launch_partial_sum(const PartSumArgs &a, hipStream_t s) {
  const int64_t total = a.T * (a.d / 4);
  if (total <= 0) return hipSuccess;
  int64_t blocks = (total + THREADS - 1) / THREADS;
  const int64_t cap = 256 * 16;  // 16 workgroups per CU on a 256-CU device
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(partial_sum_kernel, dim3((unsigned)blocks), dim3(THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace tpmlp
