// fp32 GEMM with the same epilogues, for the fp32 variant of the shard (the Day
// 41 post checks its column split in fp32).  Correctness first: every output
// element is one thread's fused multiply-add chain over k in ascending order,
// so the value of an element does not depend on which tile or shard computed
// it, and a column-split result concatenates bit-exactly into the unsplit one.
#include "device_common.hpp"
#include "kernels.h"

namespace tpmlp {
namespace {

constexpr int TS = 16;  // 16 x 16 outputs per workgroup, 16-k LDS steps

template <int EPI, int ACT, int LAY>
__global__ __launch_bounds__(TS *TS) void gemm_f32_kernel(const GemmArgs p) {
  constexpr bool DUAL = (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_SAVE);
  __shared__ float As[TS][TS + 1];
  __shared__ float Bs[TS][TS + 1];
  __shared__ float B2s[DUAL ? TS : 1][TS + 1];

  const int g = blockIdx.z;
  const float *A = (const float *)p.A + g * p.sA;
  const float *B = (const float *)p.B + g * p.sB;
  const float *B2 = DUAL ? (const float *)p.B2 + g * p.sB2 : nullptr;
  const int tx = threadIdx.x % TS, ty = threadIdx.x / TS;
  const int64_t row = (int64_t)blockIdx.y * TS + ty, col = (int64_t)blockIdx.x * TS + tx;
  float acc = 0.0f, acc2 = 0.0f;
  for (int64_t k0 = 0; k0 < p.K; k0 += TS) {
    const int64_t ka = k0 + tx, kb = k0 + ty;
    // A (m, k) at A[m lda + k], or at A[k lda + m] when A is held transposed;
    // B (k, n) at B[k ldb + n], or at B[n ldb + k] when held transposed.
    if constexpr (LAY == LAY_TN) {
      const int64_t ar = (int64_t)blockIdx.y * TS + tx, ak = k0 + ty;  // coalesced along m
      As[tx][ty] = (ar < p.M && ak < p.K) ? A[ak * p.lda + ar] : 0.0f;
    } else {
      As[ty][tx] = (row < p.M && ka < p.K) ? A[row * p.lda + ka] : 0.0f;
    }
    if constexpr (LAY == LAY_NT) {
      const int64_t bc = (int64_t)blockIdx.x * TS + ty, bk = k0 + tx;  // coalesced along k
      // k past ksplit comes from the second matrix (same leading dimension)
      const bool second = p.ksplit > 0 && bk >= p.ksplit;
      const float *Bk = second ? (const float *)p.B2 : B;
      const int64_t kq = second ? bk - p.ksplit : bk;
      Bs[tx][ty] = (bc < p.N && bk < p.K) ? Bk[src_col(p, bc) * p.ldb + kq] : 0.0f;
    } else {
      Bs[ty][tx] = (col < p.N && kb < p.K) ? B[kb * p.ldb + src_col(p, col)] : 0.0f;
    }
    if (DUAL) B2s[ty][tx] = (col < p.N && kb < p.K) ? B2[kb * p.ldb2 + col] : 0.0f;
    __syncthreads();
    const int kn = (p.K - k0) < TS ? (int)(p.K - k0) : TS;
    for (int kk = 0; kk < kn; ++kk) {
      acc = fmaf(As[ty][kk], Bs[kk][tx], acc);
      if (DUAL) acc2 = fmaf(As[ty][kk], B2s[kk][tx], acc2);
    }
    __syncthreads();
  }
  if (row >= p.M || col >= p.N) return;
  float *C = (float *)p.C + g * p.sC;
  float *C2 = (float *)p.C2;
  const float *H = (const float *)p.aux;
  if constexpr (EPI == EPI_F32) {
    C[row * p.ldc + col] = acc;
  } else if constexpr (EPI == EPI_F32_ACC) {
    C[row * p.ldc + col] += acc;
  } else if constexpr (DUAL) {
    C[row * p.ldc + col] = silu(acc) * acc2;
    if constexpr (EPI == EPI_SWIGLU_SAVE) {
      C2[row * p.ldc2 + col] = acc;
      C2[row * p.ldc2 + p.N + col] = acc2;
    }
  } else if constexpr (EPI == EPI_DACT) {
    C[row * p.ldc + col] = acc * dactivate<ACT>(H[row * p.ldaux + col]);
  } else if constexpr (EPI == EPI_DSWIGLU) {
    const float gv = H[row * p.ldaux + col], uv = H[row * p.ldaux + p.N + col];
    C[row * p.ldc + col] = acc * uv * dactivate<ACT_SWIGLU>(gv);
    C[row * p.ldc + p.N + col] = acc * silu(gv);
  } else {
    const float bv = p.bias ? ((const float *)p.bias + g * p.sBias)[src_col(p, col)] : 0.0f;
    C[row * p.ldc + col] = activate<ACT>(acc + bv);
    if constexpr (EPI == EPI_ACT_SAVE) C2[row * p.ldc2 + col] = acc + bv;
  }
}

template <int EPI, int ACT, int LAY>
hipError_t launch_t(const GemmArgs &a, hipStream_t s) {
  const int64_t gx = (a.N + TS - 1) / TS, gy = (a.M + TS - 1) / TS;
  if (gx <= 0 || gy <= 0 || a.groups <= 0) return hipSuccess;
  if (gx > 0x7fffffff || gy > 65535 || a.groups > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_f32_kernel<EPI, ACT, LAY>), dim3((unsigned)gx, (unsigned)gy, a.groups),
                     dim3(TS * TS), 0, s, a);
  return hipGetLastError();
}

template <int EPI, int LAY>
hipError_t launch_act(const GemmArgs &a, hipStream_t s) {
  switch (a.act) {
    case ACT_NONE:
      return launch_t<EPI, ACT_NONE, LAY>(a, s);
    case ACT_RELU:
      return launch_t<EPI, ACT_RELU, LAY>(a, s);
    case ACT_GELU_TANH:
      return launch_t<EPI, ACT_GELU_TANH, LAY>(a, s);
    case ACT_GELU_ERF:
      return launch_t<EPI, ACT_GELU_ERF, LAY>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm_f32(const GemmArgs &a, hipStream_t s) {
  if (a.lay == LAY_NN) {
    switch (a.epi) {
      case EPI_F32:
        return launch_t<EPI_F32, ACT_NONE, LAY_NN>(a, s);
      case EPI_SWIGLU:
        return launch_t<EPI_SWIGLU, ACT_SWIGLU, LAY_NN>(a, s);
      case EPI_SWIGLU_SAVE:
        return launch_t<EPI_SWIGLU_SAVE, ACT_SWIGLU, LAY_NN>(a, s);
      case EPI_ACT:
        return launch_act<EPI_ACT, LAY_NN>(a, s);
      case EPI_ACT_SAVE:
        return launch_act<EPI_ACT_SAVE, LAY_NN>(a, s);
    }
  } else if (a.lay == LAY_NT) {
    switch (a.epi) {
      case EPI_F32:
        return launch_t<EPI_F32, ACT_NONE, LAY_NT>(a, s);
      case EPI_F32_ACC:
        return launch_t<EPI_F32_ACC, ACT_NONE, LAY_NT>(a, s);
      case EPI_DACT:
        return launch_act<EPI_DACT, LAY_NT>(a, s);
      case EPI_DSWIGLU:
        return launch_t<EPI_DSWIGLU, ACT_SWIGLU, LAY_NT>(a, s);
    }
  } else if (a.lay == LAY_TN && a.epi == EPI_F32) {
    return launch_t<EPI_F32, ACT_NONE, LAY_TN>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tpmlp
