// The row step between the two halves of a transformer block and after it
// ("Building GPT from Scratch, Part 9", section "Communication Pattern per
// Transformer Block": the attention and the FFN each end in an all-reduce of
// the row-parallel partials, then the residual is added; each half starts
// with a LayerNorm that every GPU applies to the whole row):
//   x = (((parts[0] + parts[1]) + ...) + bias) + R     fp32, left to right,
//                                                      absent terms skipped
//   X = x                                              if X is given
//   A = (x - mean) / sqrt(var + eps) * gamma + beta    bf16, if gamma is given
// with the mean and the biased variance over the row's d elements.
//
// HBM-bound: one workgroup of 256 threads per row; each thread holds NCH
// 16-byte chunks of the row in registers, so every term is read once (the
// loads of one term for all chunks are issued together before they are
// added), the row sum and the sum of squared deviations come from two
// reductions over registers (wave shuffles, then the 4 waves through LDS),
// and X and A are written once.  The partials are read once and carry the
// nontemporal hint; the residual and the bias are ordinary loads.
#include "device_common.hpp"
#include "kernels.h"

namespace tpmlp {
namespace {

constexpr int THREADS = 256;

// Sum over the workgroup, returned to every thread.  `red` holds 4 floats.
__device__ __forceinline__ float wg_sum(float x, float *red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = x;
  __syncthreads();
  const float t = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();  // `red` is reused by the next reduction
  return t;
}

template <int NCH>
__global__ __launch_bounds__(THREADS) void residual_ln_kernel(const RowNormArgs a) {
  __shared__ float red[4];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t d4 = a.d / 4;
  f32x4 v[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) v[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  bool first = true;
  // Adds one term (a row of `base`, 4-float chunks); the first term is taken
  // as it is, so the sum equals a left-to-right fp32 sum bit for bit.
  auto add = [&](const float *base, bool nt) {
    f32x4 x[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int64_t q = tid + (int64_t)THREADS * c;
      if (q < d4)
        x[c] = nt ? __builtin_nontemporal_load((const f32x4 *)(base + 4 * q))
                  : *(const f32x4 *)(base + 4 * q);
      else
        x[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c) v[c] = first ? x[c] : v[c] + x[c];
    first = false;
  };
  for (int s = 0; s < a.p; ++s) add(a.parts[s] + t * a.ldp, true);
  if (a.bias) add(a.bias, false);
  if (a.R) add(a.R + t * a.ldr, false);

  if (a.X) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int64_t q = tid + (int64_t)THREADS * c;
      if (q < d4) *(f32x4 *)(a.X + t * a.ldx + 4 * q) = v[c];
    }
  }
  if (!a.gamma) return;

  float s1 = 0.0f;
#pragma unroll
  for (int c = 0; c < NCH; ++c)
    if (tid + (int64_t)THREADS * c < d4) s1 += (v[c][0] + v[c][1]) + (v[c][2] + v[c][3]);
  const float mean = wg_sum(s1, red) / (float)a.d;
  float s2 = 0.0f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (tid + (int64_t)THREADS * c < d4) {
      const f32x4 e = v[c] - mean;
      s2 += (e[0] * e[0] + e[1] * e[1]) + (e[2] * e[2] + e[3] * e[3]);
    }
  }
  const float var = wg_sum(s2, red) / (float)a.d;
  const float rstd = 1.0f / sqrtf(var + a.eps);
  bf16 *A = (bf16 *)a.A + t * a.lda;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int64_t q = tid + (int64_t)THREADS * c;
    if (q < d4) {
      const f32x4 g = *(const f32x4 *)(a.gamma + 4 * q);
      const f32x4 b = *(const f32x4 *)(a.beta + 4 * q);
      const f32x4 y = (v[c] - mean) * rstd * g + b;
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      *(bf16x4 *)(A + 4 * q) = bf16x4{to_bf16(y[0]), to_bf16(y[1]), to_bf16(y[2]), to_bf16(y[3])};
    }
  }
}

template <int NCH>
hipError_t launch_n(const RowNormArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(residual_ln_kernel<NCH>, dim3((unsigned)a.T), dim3(THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_residual_ln(const RowNormArgs &a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  if (a.T > 0x7fffffff || a.d < 4 || a.d % 4 || a.d > kRowNormMaxD) return hipErrorInvalidValue;
  const int64_t chunks = (a.d / 4 + THREADS - 1) / THREADS;  // 16-byte chunks per thread
  if (chunks <= 1) return launch_n<1>(a, s);
  if (chunks <= 2) return launch_n<2>(a, s);
  if (chunks <= 4) return launch_n<4>(a, s);
  if (chunks <= 8) return launch_n<8>(a, s);
  return launch_n<16>(a, s);
}

}  // namespace tpmlp
