// Few-token (T <= 64) bf16 GEMM for gfx950: the decode regime, where each
// shard's weights are read once per step and HBM bandwidth sets the time.
// ("What is Tensor Parallelism?", Llama 3.1 70B worked example: a decode token
// is tiny next to the 3584-column weight shard every GPU streams.)
//
// Work split: a workgroup owns a block of 128 "virtual" output columns and one
// of S contiguous k-ranges; its 4 waves take the 32-k steps of that range in
// turn.  Per step a lane loads an 8(k) x 8(n) bf16 block of the weight (eight
// 16-byte row loads; 16 lanes cover 256 contiguous bytes of a row), transposes
// it in registers into eight 8-k vectors and feeds eight
// v_mfma_f32_16x16x32_bf16 (M = tokens padded to 16), so MFMA column c of
// product j is weight column 8c + j of the block.  For SwiGLU lanes 0..7 of
// each 16 read the gate matrix and lanes 8..15 the up matrix (64 output
// columns per block); the epilogue swaps halves between lanes.
//
// Reduction: waves sum through LDS in a fixed order; with S > 1 the workgroup
// partial goes to the workspace, and the last workgroup to arrive on a column
// block (an atomic counter) sums the S partials in k-range order and applies
// the epilogue, then zeroes the counter.  The result therefore does not depend
// on arrival order.
#include "device_common.hpp"
#include "kernels.h"

namespace tpmlp {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int NW = 4;          // waves per workgroup
constexpr int KSTEP = 32;      // k per MFMA step
constexpr int VCOLS = 128;     // virtual columns per workgroup
constexpr int MIN_STEPS_PER_WAVE = 4;
constexpr int TARGET_WGS = 1024;

struct DecodePlan {
  int64_t nblk;    // column blocks
  int64_t S;       // k-ranges (split-K factor)
  int64_t kc;      // k per range (multiple of KSTEP)
  int mb;          // 16-row M blocks (1, 2 or 4)
  bool dual;
};

DecodePlan make_plan(const GemmArgs &a) {
  DecodePlan pl;
  pl.dual = a.epi == EPI_SWIGLU;
  const int64_t width = pl.dual ? VCOLS / 2 : VCOLS;
  pl.nblk = (a.N + width - 1) / width;
  pl.mb = a.M <= 16 ? 1 : (a.M <= 32 ? 2 : 4);
  const int64_t steps = (a.K + KSTEP - 1) / KSTEP;
  int64_t S = (TARGET_WGS + pl.nblk - 1) / pl.nblk;
  int64_t smax = steps / (NW * MIN_STEPS_PER_WAVE);
  if (smax < 1) smax = 1;
  if (S > smax) S = smax;
  if (S < 1) S = 1;
  const int64_t steps_per = (steps + S - 1) / S;
  pl.kc = steps_per * KSTEP;
  pl.S = (a.K + pl.kc - 1) / pl.kc;
  return pl;
}

constexpr size_t kCounterAlign = 256;

size_t counters_bytes(const DecodePlan &pl) {
  return ((size_t)pl.nblk * sizeof(unsigned) + kCounterAlign - 1) / kCounterAlign * kCounterAlign;
}

size_t plan_ws_bytes(const DecodePlan &pl) {
  if (pl.S <= 1) return 0;
  return counters_bytes(pl) + (size_t)pl.nblk * pl.S * pl.mb * 32 * 64 * sizeof(float);
}

template <int EPI, int ACT, int MB>
__global__ __launch_bounds__(NW * 64) void gemm_bf16_decode_kernel(const GemmArgs p, int64_t nblk,
                                                                   int64_t S, int64_t kc,
                                                                   unsigned *counters,
                                                                   float *parts) {
  constexpr bool DUAL = (EPI == EPI_SWIGLU);
  constexpr int NACC = MB * 8;
  __shared__ float red[(NW - 1) * 32 * 64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t blk = blockIdx.x % nblk, s = blockIdx.x / nblk;
  const int cb = lane & 15, kq = lane >> 4;
  const int64_t M = p.M, N = p.N, K = p.K;

  // Which weight matrix and column group this lane streams.
  const bf16 *W;
  int64_t ldw, col;
  if (DUAL) {
    const bool up = cb >= 8;
    W = (const bf16 *)(up ? p.B2 : p.B);
    ldw = up ? p.ldb2 : p.ldb;
    col = blk * (VCOLS / 2) + 8 * (cb & 7);
  } else {
    W = (const bf16 *)p.B;
    ldw = p.ldb;
    col = blk * VCOLS + 8 * cb;
  }
  const bool col_ok = col < N;
  const bf16 *X = (const bf16 *)p.A;

  f32x4 acc[NACC];
#pragma unroll
  for (int e = 0; e < NACC; ++e) acc[e] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const int64_t kbeg = s * kc;
  const int64_t kend = (kbeg + kc < K) ? kbeg + kc : K;
  const u32x4 z4 = {0u, 0u, 0u, 0u};

  for (int64_t k0 = kbeg + (int64_t)wave * KSTEP; k0 < kend; k0 += NW * KSTEP) {
    const int64_t kr = k0 + 8 * kq;  // this lane's 8-row k chunk
    const bool k_ok = kr < kend;     // K and kend are multiples of 8
    u32x4 w[8];
#pragma unroll
    for (int r = 0; r < 8; ++r)
      w[r] = (col_ok && k_ok) ? *(const u32x4 *)(W + (kr + r) * ldw + col) : z4;
    u32x4 xa[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const int64_t row = 16 * m + cb;
      xa[m] = (row < M && k_ok) ? *(const u32x4 *)(X + row * p.lda + kr) : z4;
    }
    // 8x8 transpose: column j of the block as 8 consecutive k (4 dwords of k pairs).
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u32x4 bt;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = w[2 * q][j >> 1], hi = w[2 * q + 1][j >> 1];
        bt[q] = (j & 1) ? pack_hi(lo, hi) : pack_lo(lo, hi);
      }
      const bf16x8 bv = __builtin_bit_cast(bf16x8, bt);
#pragma unroll
      for (int m = 0; m < MB; ++m)
        acc[m * 8 + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, xa[m]), bv, acc[m * 8 + j], 0, 0, 0);
    }
  }

  // Sum the waves in LDS, wave 0 first, in chunks of 8 accumulators.
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    if (wave > 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[((wave - 1) * 32 + j * 4 + v) * 64 + lane] = acc[m * 8 + j][v];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int w2 = 0; w2 < NW - 1; ++w2)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[m * 8 + j][v] += red[(w2 * 32 + j * 4 + v) * 64 + lane];
    }
    __syncthreads();
  }
  if (wave != 0) return;

  if (S > 1) {
    float *mine = parts + (size_t)(blk * S + s) * (MB * 32 * 64);
#pragma unroll
    for (int e = 0; e < NACC; ++e)
#pragma unroll
      for (int v = 0; v < 4; ++v) mine[(e * 4 + v) * 64 + lane] = acc[e][v];
    __threadfence();
    unsigned old = 0;
    if (lane == 0) old = atomicAdd(&counters[blk], 1u);
    old = __shfl(old, 0);
    if (old != (unsigned)(S - 1)) return;
    __threadfence();
    const float *base = parts + (size_t)blk * S * (MB * 32 * 64);
#pragma unroll
    for (int e = 0; e < NACC; ++e)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[e][v] = base[(e * 4 + v) * 64 + lane];
    for (int64_t s2 = 1; s2 < S; ++s2) {
      const float *ps = base + (size_t)s2 * (MB * 32 * 64);
#pragma unroll
      for (int e = 0; e < NACC; ++e)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[e][v] += ps[(e * 4 + v) * 64 + lane];
    }
    if (lane == 0) atomicExch(&counters[blk], 0u);
  }

  // Epilogue.  16x16 accumulator layout: lane holds MFMA column (lane & 15) and
  // rows 4 (lane / 16) + v, v = 0..3; product j's column c is block column 8c + j.
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t row = 16 * m + 4 * kq + v;
        const float val = acc[m * 8 + j][v];
        if constexpr (DUAL) {
          const float other = __shfl_xor(val, 8);
          if (cb < 8 && col_ok && row < M) {
            bf16 *C = (bf16 *)p.C;
            C[row * p.ldc + col + j] = to_bf16(silu(val) * other);
          }
        } else if constexpr (EPI == EPI_F32) {
          if (col_ok && row < M) ((float *)p.C)[row * p.ldc + col + j] = val;
        } else {
          if (col_ok && row < M) {
            const float bv = p.bias ? (float)((const bf16 *)p.bias)[col + j] : 0.0f;
            ((bf16 *)p.C)[row * p.ldc + col + j] = to_bf16(activate<ACT>(val + bv));
          }
        }
      }
}

template <int EPI, int ACT>
hipError_t launch_mb(const GemmArgs &a, const DecodePlan &pl, void *ws, hipStream_t st) {
  unsigned *counters = (unsigned *)ws;
  float *parts = pl.S > 1 ? (float *)((char *)ws + counters_bytes(pl)) : nullptr;
  const dim3 grid((unsigned)(pl.nblk * pl.S)), block(NW * 64);
  switch (pl.mb) {
    case 1:
      hipLaunchKernelGGL((gemm_bf16_decode_kernel<EPI, ACT, 1>), grid, block, 0, st, a, pl.nblk,
                         pl.S, pl.kc, counters, parts);
      break;
    case 2:
      hipLaunchKernelGGL((gemm_bf16_decode_kernel<EPI, ACT, 2>), grid, block, 0, st, a, pl.nblk,
                         pl.S, pl.kc, counters, parts);
      break;
    default:
      hipLaunchKernelGGL((gemm_bf16_decode_kernel<EPI, ACT, 4>), grid, block, 0, st, a, pl.nblk,
                         pl.S, pl.kc, counters, parts);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_one(const GemmArgs &a, void *ws, hipStream_t st) {
  const DecodePlan pl = make_plan(a);
  switch (a.epi) {
    case EPI_F32:
      return launch_mb<EPI_F32, ACT_NONE>(a, pl, ws, st);
    case EPI_SWIGLU:
      return launch_mb<EPI_SWIGLU, ACT_SWIGLU>(a, pl, ws, st);
    case EPI_ACT:
      switch (a.act) {
        case ACT_NONE:
          return launch_mb<EPI_ACT, ACT_NONE>(a, pl, ws, st);
        case ACT_RELU:
          return launch_mb<EPI_ACT, ACT_RELU>(a, pl, ws, st);
        case ACT_GELU_TANH:
          return launch_mb<EPI_ACT, ACT_GELU_TANH>(a, pl, ws, st);
        case ACT_GELU_ERF:
          return launch_mb<EPI_ACT, ACT_GELU_ERF>(a, pl, ws, st);
      }
  }
  return hipErrorInvalidValue;
}

}  // namespace

size_t decode_workspace_bytes(const GemmArgs &a) { return plan_ws_bytes(make_plan(a)); }

hipError_t launch_gemm_bf16_decode(const GemmArgs &a, void *ws, hipStream_t st) {
  if (a.M <= 0 || a.M > 64) return hipErrorInvalidValue;
  // Groups run one after another on the stream; they share the workspace.
  for (int g = 0; g < a.groups; ++g) {
    GemmArgs one = a;
    one.groups = 1;
    one.A = (const bf16 *)a.A + g * a.sA;
    one.B = (const bf16 *)a.B + g * a.sB;
    one.B2 = a.B2 ? (const void *)((const bf16 *)a.B2 + g * a.sB2) : nullptr;
    one.bias = a.bias ? (const void *)((const bf16 *)a.bias + g * a.sBias) : nullptr;
    if (a.epi == EPI_F32)
      one.C = (float *)a.C + g * a.sC;
    else
      one.C = (bf16 *)a.C + g * a.sC;
    const hipError_t e = launch_one(one, ws, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tpmlp
