// Few-token (T <= 64) bf16 GEMM for gfx950: the decode regime, where each
// shard's weights are read once per step and HBM bandwidth sets the time.
// ("What is Tensor Parallelism?", Llama 3.1 70B worked example: a decode token
// is tiny next to the 3584-column weight shard every GPU streams.)
//
// Weight streaming.  A workgroup owns a block of 128 "virtual" output columns
// and one of S contiguous k-ranges; its waves take the 32-k steps of that
// range in turn (8 waves; 4 for more than 32 tokens).  Per step a lane loads an 8(k) x 8(n) bf16 block of the
// weight (eight 16-byte row loads; 16 lanes cover 256 contiguous bytes of a
// row), transposes it in registers into eight 8-k vectors and feeds eight
// v_mfma_f32_16x16x32_bf16 (M = tokens padded to 16), so MFMA column c of
// product j is weight column 8c + j of the block.  A ring of register buffers
// keeps the loads of the next 2-3 steps in flight while one step is
// transposed and multiplied.
// For SwiGLU lanes 0..7 of each 16 read the gate matrix and lanes 8..15 the up
// matrix (64 output columns per block); the epilogue swaps halves between
// lanes.
//
// Reduction.  The waves of a workgroup are summed through LDS in a fixed
// order.  With S = 1 the workgroup applies the epilogue itself; with S > 1 it
// writes its partial to the workspace and a second kernel sums the S partials
// of each column block in k-range order and applies the epilogue.  Either way
// the result does not depend on timing, and no inter-workgroup
// synchronisation is needed inside a kernel.
#include <cstdlib>

#include "device_common.hpp"
#include "kernels.h"

namespace tpmlp {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16 zero bytes that masked-off lanes load instead of matrix data.
__device__ __attribute__((aligned(16))) u32x4 g_zero16;

// Waves per workgroup and depth of the register ring, by 16-row M blocks:
// more tokens need more accumulators, so fewer buffers fit (two waves per SIMD
// share 512 registers; one wave per SIMD has them all).
constexpr int nw_for(int mb) { return mb >= 4 ? 4 : 8; }
constexpr int nbuf_for(int mb) { return mb >= 4 ? 3 : (mb == 2 ? 3 : 4); }
constexpr int KSTEP = 32;      // k per MFMA step
constexpr int VCOLS = 128;     // virtual columns per workgroup
// One workgroup fills a CU (its waves hold most of the register file), so
// the split is chosen to give at most one workgroup per CU of a 256-CU device.
constexpr int TARGET_WGS = 256;
constexpr int MIN_STEPS_PER_WAVE = 4;

struct DecodePlan {
  int64_t nblk;  // column blocks
  int64_t S;     // k-ranges (split-K factor)
  int64_t kc;    // k per range (multiple of KSTEP)
  int mb;        // 16-row M blocks (1, 2 or 4)
};

int split_override() {
  static int v = [] {
    const char *e = getenv("TPMLP_DECODE_SPLIT");
    return e ? atoi(e) : 0;
  }();
  return v;
}

DecodePlan make_plan(const GemmArgs &a) {
  DecodePlan pl;
  const bool dual = a.epi == EPI_SWIGLU;
  const int64_t width = dual ? VCOLS / 2 : VCOLS;
  pl.nblk = (a.N + width - 1) / width;
  pl.mb = a.M <= 16 ? 1 : (a.M <= 32 ? 2 : 4);
  const int64_t steps = (a.K + KSTEP - 1) / KSTEP;
  int64_t S = TARGET_WGS / pl.nblk;
  int64_t smax = steps / (nw_for(pl.mb) * MIN_STEPS_PER_WAVE);
  if (smax < 1) smax = 1;
  if (S > smax) S = smax;
  if (S < 1) S = 1;
  if (split_override() > 0) S = split_override();
  const int64_t steps_per = (steps + S - 1) / S;
  pl.kc = steps_per * KSTEP;
  pl.S = (a.K + pl.kc - 1) / pl.kc;
  return pl;
}

constexpr int64_t part_floats(int mb) { return (int64_t)mb * 32 * 64; }

size_t plan_ws_bytes(const DecodePlan &pl) {
  if (pl.S <= 1) return 0;
  return (size_t)pl.nblk * pl.S * part_floats(pl.mb) * sizeof(float);
}

// Epilogue of one accumulator set: rows 16 m + 4 kq + v, block column
// 8 cb + j (SwiGLU: cb < 8 gate, cb >= 8 up of the same column).
template <int EPI, int ACT, int MB>
__device__ __forceinline__ void decode_epilogue(const GemmArgs &p, int64_t blk, int lane,
                                                const f32x4 (&acc)[MB * 8]) {
  constexpr bool DUAL = (EPI == EPI_SWIGLU);
  const int cb = lane & 15, kq = lane >> 4;
  const int64_t col = DUAL ? blk * (VCOLS / 2) + 8 * (cb & 7) : blk * VCOLS + 8 * cb;
  const bool col_ok = col < p.N;
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
          if (cb < 8 && col_ok && row < p.M)
            ((bf16 *)p.C)[row * p.ldc + col + j] = to_bf16(silu(val) * other);
        } else if constexpr (EPI == EPI_F32) {
          if (col_ok && row < p.M) ((float *)p.C)[row * p.ldc + col + j] = val;
        } else {
          if (col_ok && row < p.M) {
            const float bv = p.bias ? (float)((const bf16 *)p.bias)[col + j] : 0.0f;
            ((bf16 *)p.C)[row * p.ldc + col + j] = to_bf16(activate<ACT>(val + bv));
          }
        }
      }
}

template <int EPI, int ACT, int MB>
__global__ __launch_bounds__(nw_for(MB) * 64) void gemm_bf16_decode_kernel(const GemmArgs p,
                                                                           int64_t nblk,
                                                                           int64_t S, int64_t kc,
                                                                           float *parts) {
  constexpr bool DUAL = (EPI == EPI_SWIGLU);
  constexpr int NACC = MB * 8;
  constexpr int NW = nw_for(MB);
  __shared__ float red[(NW - 1) * 32 * 64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  // Loads of the step starting at k0 (its 8 weight rows and the X chunks).
  // Every load is issued: a lane outside the matrix reads 16 zero bytes from
  // g_zero16 instead, so the value needs no select and no branch surrounds a
  // load (g_zero16 is not const, so its contents cannot be assumed).
  const u32x4 *zero = &g_zero16;
  // The empty asm hides where the selected address came from, so the compiler
  // cannot turn "load from one of two addresses" back into a branch.
  typedef __attribute__((address_space(1))) const u32x4 gu32x4;
  auto load16 = [&](bool ok, const bf16 *ptr) {
    gu32x4 *q = (gu32x4 *)(ok ? (const u32x4 *)ptr : zero);
    asm volatile("" : "+v"(q));
    return *q;
  };
  auto load_step = [&](int64_t k0, u32x4(&w)[8], u32x4(&xa)[MB]) {
    const int64_t kr = k0 + 8 * kq;  // this lane's 8-row k chunk
    const bool ok = col_ok && kr < kend;  // K and kend are multiples of 8
#pragma unroll
    for (int r = 0; r < 8; ++r) w[r] = load16(ok, W + (kr + r) * ldw + col);
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const int64_t row = 16 * m + cb;
      xa[m] = load16(row < M && kr < kend, X + row * p.lda + kr);
    }
  };
  // 8x8 transpose (column j of the block as 8 consecutive k) and the MFMAs.
  auto compute_step = [&](const u32x4(&w)[8], const u32x4(&xa)[MB]) {
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
  };

  // Steps of this wave: kbeg + (wave + NW i) * KSTEP.  A ring of NBUF
  // register buffers keeps NBUF-1 steps of loads in flight while one step is
  // transposed and multiplied.  The trip count is uniform and every load is
  // issued (lanes past kend load nothing and get zeros), so the loop has no
  // data-dependent branch and the waits stay exact.
  constexpr int NBUF = nbuf_for(MB);
  const int64_t kstride = (int64_t)NW * KSTEP;
  const int64_t k0 = kbeg + (int64_t)wave * KSTEP;
  const int64_t nsteps = (kend - kbeg + kstride - 1) / kstride;  // steps of wave 0
  const int64_t iters = (nsteps + NBUF - 1) / NBUF;
  u32x4 wb[NBUF][8], xb[NBUF][MB];
#pragma unroll
  for (int b = 0; b < NBUF - 1; ++b) load_step(k0 + b * kstride, wb[b], xb[b]);
  for (int64_t it = 0; it < iters; ++it) {
    const int64_t kb = k0 + it * NBUF * kstride;
#pragma unroll
    for (int b = 0; b < NBUF; ++b) {
      const int nb = (b + NBUF - 1) % NBUF;
      load_step(kb + (b + NBUF - 1) * kstride, wb[nb], xb[nb]);
      compute_step(wb[b], xb[b]);
    }
  }

  // Sum the waves in LDS, wave 0 first, in chunks of 8 accumulators.
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    if (wave > 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          red[((wave - 1) * 32 + j * 4 + v) * 64 + lane] = acc[m * 8 + j][v];
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
    float *mine = parts + (blk * S + s) * part_floats(MB);
#pragma unroll
    for (int e = 0; e < NACC; ++e)
#pragma unroll
      for (int v = 0; v < 4; ++v) mine[(e * 4 + v) * 64 + lane] = acc[e][v];
    return;
  }
  decode_epilogue<EPI, ACT, MB>(p, blk, lane, acc);
}

// Sum of the S partials of each column block (k-range order) and epilogue.
// One thread per 4 consecutive partial floats (one lane, one accumulator
// register e, v = 0..3); for SwiGLU it also takes the matching up value
// (lane ^ 8), so each thread owns whole output elements.  All S loads of a
// thread are issued before they are added.
template <int EPI, int ACT, int MB>
__global__ __launch_bounds__(256) void decode_reduce_kernel(const GemmArgs p, int64_t nblk,
                                                            int64_t S, const float *parts) {
  constexpr bool DUAL = (EPI == EPI_SWIGLU);
  constexpr int PER_BLK = MB * 8 * 64;  // (e, lane) pairs per block
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= nblk * PER_BLK) return;
  const int64_t blk = t / PER_BLK;
  const int idx = (int)(t - blk * PER_BLK);
  const int e = idx / 64, lane = idx % 64;
  const int cb = lane & 15, kq = lane >> 4;
  if (DUAL && cb >= 8) return;  // handled together with its gate lane
  const int m = e / 8, j = e % 8;
  const float *base = parts + blk * S * part_floats(MB);
  f32x4 a = {0.0f, 0.0f, 0.0f, 0.0f}, u = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int64_t s2 = 0; s2 < S; ++s2) {
    const float *ps = base + s2 * part_floats(MB);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      a[v] += ps[(e * 4 + v) * 64 + lane];
      if (DUAL) u[v] += ps[(e * 4 + v) * 64 + (lane ^ 8)];
    }
  }
  const int64_t col = DUAL ? blk * (VCOLS / 2) + 8 * cb + j : blk * VCOLS + 8 * cb + j;
  if (col >= p.N) return;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t row = 16 * m + 4 * kq + v;
    if (row >= p.M) continue;
    if constexpr (DUAL) {
      ((bf16 *)p.C)[row * p.ldc + col] = to_bf16(silu(a[v]) * u[v]);
    } else if constexpr (EPI == EPI_F32) {
      ((float *)p.C)[row * p.ldc + col] = a[v];
    } else {
      const float bv = p.bias ? (float)((const bf16 *)p.bias)[col] : 0.0f;
      ((bf16 *)p.C)[row * p.ldc + col] = to_bf16(activate<ACT>(a[v] + bv));
    }
  }
}

template <int EPI, int ACT, int MB>
hipError_t launch_plan(const GemmArgs &a, const DecodePlan &pl, void *ws, hipStream_t st) {
  float *parts = pl.S > 1 ? (float *)ws : nullptr;
  hipLaunchKernelGGL((gemm_bf16_decode_kernel<EPI, ACT, MB>), dim3((unsigned)(pl.nblk * pl.S)),
                     dim3(nw_for(MB) * 64), 0, st, a, pl.nblk, pl.S, pl.kc, parts);
  if (pl.S > 1) {
    const int64_t threads = pl.nblk * MB * 8 * 64;
    hipLaunchKernelGGL((decode_reduce_kernel<EPI, ACT, MB>), dim3((unsigned)((threads + 255) / 256)),
                       dim3(256), 0, st, a, pl.nblk, pl.S, (const float *)parts);
  }
  return hipGetLastError();
}

template <int EPI, int ACT>
hipError_t launch_mb(const GemmArgs &a, const DecodePlan &pl, void *ws, hipStream_t st) {
  switch (pl.mb) {
    case 1:
      return launch_plan<EPI, ACT, 1>(a, pl, ws, st);
    case 2:
      return launch_plan<EPI, ACT, 2>(a, pl, ws, st);
    default:
      return launch_plan<EPI, ACT, 4>(a, pl, ws, st);
  }
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
