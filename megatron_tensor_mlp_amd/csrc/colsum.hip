// Column sums of a [T, n] matrix in fp32, for the bias gradient of the column
// step (the sum over tokens of the hidden gradient).  Two passes, so that the
// order of the additions is fixed: pass 1 sums chunks of CH consecutive rows
// of each column (rows ascending) into a [chunks, n] fp32 workspace; pass 2
// adds the chunk sums of each column in chunk order.  Both passes read along
// rows, one column per lane, so every load instruction covers consecutive
// columns.  HBM-bound and small next to the GEMMs around it.
#include "device_common.hpp"
#include "kernels.h"

namespace tpmlp {
namespace {

constexpr int CH = 64;    // rows per chunk
constexpr int TPB = 256;  // columns per workgroup

template <typename E>
__global__ __launch_bounds__(TPB) void colsum_chunks(const E *H, int64_t ldh, int64_t T, int64_t n,
                                                     float *part) {
  const int64_t col = (int64_t)blockIdx.x * TPB + threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.y * CH;
  if (col >= n) return;
  const int64_t rows = (T - r0) < CH ? (T - r0) : CH;
  float v[CH];
#pragma unroll
  for (int r = 0; r < CH; ++r) v[r] = r < rows ? (float)H[(r0 + r) * ldh + col] : 0.0f;
  float acc = v[0];
#pragma unroll
  for (int r = 1; r < CH; ++r)
    if (r < rows) acc += v[r];
  part[(int64_t)blockIdx.y * n + col] = acc;
}

__global__ __launch_bounds__(TPB) void colsum_final(const float *part, int64_t chunks, int64_t n,
                                                    float *out) {
  const int64_t col = (int64_t)blockIdx.x * TPB + threadIdx.x;
  if (col >= n) return;
  float acc = 0.0f;
  for (int64_t c = 0; c < chunks; ++c) acc = (c == 0) ? part[col] : acc + part[c * n + col];
  out[col] = acc;
}

}  // namespace

size_t colsum_workspace_bytes(int64_t T, int64_t n) {
  const int64_t chunks = (T + CH - 1) / CH;
  return (size_t)(chunks > 0 ? chunks : 0) * (size_t)n * sizeof(float);
}

hipError_t launch_colsum(bool bf16_in, const void *H, int64_t ldh, int64_t T, int64_t n, float *ws,
                         float *out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t chunks = (T + CH - 1) / CH;
  const int64_t gx = (n + TPB - 1) / TPB;
  if (gx > 0x7fffffff || chunks > 65535) return hipErrorInvalidValue;
  if (chunks == 0) {  // no rows: the final pass writes zeros (reads nothing)
    hipLaunchKernelGGL(colsum_final, dim3((unsigned)gx), dim3(TPB), 0, s, ws, chunks, n, out);
    return hipGetLastError();
  }
  if (bf16_in)
    hipLaunchKernelGGL(colsum_chunks<bf16>, dim3((unsigned)gx, (unsigned)chunks), dim3(TPB), 0, s,
                       (const bf16 *)H, ldh, T, n, ws);
  else
    hipLaunchKernelGGL(colsum_chunks<float>, dim3((unsigned)gx, (unsigned)chunks), dim3(TPB), 0, s,
                       (const float *)H, ldh, T, n, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(colsum_final, dim3((unsigned)gx), dim3(TPB), 0, s, ws, chunks, n, out);
  return hipGetLastError();
}

}  // namespace tpmlp
