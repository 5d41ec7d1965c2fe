// bf16 MFMA GEMM with fp32 accumulation and fused epilogues, for gfx950.
//
// Used for the column step (X * W1_i with bias + GeLU/ReLU, or the SwiGLU
// pair X * Wg_i, X * Wu_i) and the row step (Y_i * W2_i -> fp32 partial) when
// the token count is large ("Transformer math: tensor parallel", sections on
// the column- and row-parallel splits; "Tensor Parallelism Explained", 2.B).
//
// Tile: 256 rows x 256 accumulator columns x 64 k per step, 512 threads
// (8 wave64s as 2 x 4), each wave owning 128 x 64 of the tile as 4 x 2 blocks
// of v_mfma_f32_32x32x16_bf16.  For SwiGLU the 256 accumulator columns are
// 128 gate columns followed by the same 128 up columns, so every lane holds the
// gate and up value of the same output element and the epilogue is local.
//
// Data path per k-step: A (row-major, k contiguous) is copied to LDS in 16-byte
// chunks.  B is row-major [K,N] (n contiguous) but MFMA wants 8 consecutive k
// per lane, so each thread loads an 8(k) x 4(n) block, transposes it in
// registers and writes four 16-byte k-runs to LDS.  Both LDS tiles are
// [row][64 k] with the 16-byte chunk index XOR-swizzled by the row, so the
// fragment reads (8 consecutive rows, same chunk) and the writes hit distinct
// banks.  LDS is double-buffered: the global loads of step t+1 are in flight
// while step t's MFMAs run, and one barrier per step separates the buffers.
#include "device_common.hpp"
#include "kernels.h"

namespace tpmlp {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 256, BN = 256, BK = 64, NTHREADS = 512;
constexpr int TILE_ELEMS = 256 * BK;  // one LDS operand tile, bf16 elements
constexpr int GROUP_M = 4;            // row-tiles walked together for L2 reuse

// 16-byte chunk swizzle inside a 128-byte LDS row.
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int r, int ch) { return r * BK + ((ch ^ swz(r)) << 3); }

// Workgroup b runs on XCD b % 8.  Give every XCD a contiguous run of the tile
// order (a bijection for any total), then walk GROUP_M row-tiles at a time so
// the tiles resident on one XCD share A and B panels in its L2.
__device__ __forceinline__ void tile_coords(int bid, int tilesM, int tilesN, int total, int &g,
                                            int &tm, int &tn) {
  const int xcd = bid & 7, idx = bid >> 3;
  const int q = total >> 3, r = total & 7;
  const int t = xcd * q + (xcd < r ? xcd : r) + idx;
  const int per = tilesM * tilesN;
  g = t / per;
  const int u = t - g * per;
  const int span = GROUP_M * tilesN;
  const int grp = u / span;
  const int first = grp * GROUP_M;
  const int gsz = (tilesM - first) < GROUP_M ? (tilesM - first) : GROUP_M;
  const int w = u - grp * span;
  tm = first + w % gsz;
  tn = w / gsz;
}

template <int EPI, int ACT>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_bf16_tiled_kernel(const GemmArgs p) {
  constexpr bool DUAL = (EPI == EPI_SWIGLU);
  constexpr int NOUT = DUAL ? BN / 2 : BN;  // output columns per tile
  __shared__ __attribute__((aligned(16))) bf16 lds[2 * 2 * TILE_ELEMS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int tilesM = (int)((p.M + BM - 1) / BM), tilesN = (int)((p.N + NOUT - 1) / NOUT);
  int g, tm, tn;
  tile_coords(blockIdx.x, tilesM, tilesN, tilesM * tilesN * p.groups, g, tm, tn);

  const bf16 *A = (const bf16 *)p.A + g * p.sA;
  const bf16 *B = (const bf16 *)p.B + g * p.sB;
  const bf16 *B2 = DUAL ? (const bf16 *)p.B2 + g * p.sB2 : nullptr;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * NOUT;

  // A loader: chunks tid + 512 j, j = 0..3 -> row (tid >> 3) + 64 j, k-chunk tid & 7.
  const int a_r = tid >> 3, a_ch = tid & 7;
  // B loader: rows 8 kb .. 8 kb + 7 of the k-step, accumulator columns 4 nq .. 4 nq + 3.
  const int b_kb = tid >> 6, b_nq = tid & 63;
  const bf16 *bsrc;
  int64_t bld, bcol;
  if (DUAL) {
    const bool up = b_nq >= 32;
    bsrc = up ? B2 : B;
    bld = up ? p.ldb2 : p.ldb;
    bcol = n0 + 4 * (b_nq & 31);
  } else {
    bsrc = B;
    bld = p.ldb;
    bcol = n0 + 4 * b_nq;
  }
  const bool bcol_ok = bcol < N;

  u32x4 ra[4];
  u32x2 rb[8];
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  const u32x2 z2 = {0u, 0u};

  auto gload = [&](int kt) {
    const int64_t k0 = (int64_t)kt * BK;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t row = m0 + a_r + 64 * j, k = k0 + 8 * a_ch;
      ra[j] = (row < M && k < K) ? *(const u32x4 *)(A + row * p.lda + k) : z4;
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int64_t k = k0 + 8 * b_kb + r;
      rb[r] = (bcol_ok && k < K) ? *(const u32x2 *)(bsrc + k * bld + bcol) : z2;
    }
  };

  auto lds_store = [&](int buf) {
    bf16 *As = lds + buf * (2 * TILE_ELEMS);
    bf16 *Bs = As + TILE_ELEMS;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = a_r + 64 * j;
      *(u32x4 *)(As + lds_off(r, a_ch)) = ra[j];
    }
    // rb[r] holds columns (0,1) in .x and (2,3) in .y of k-row r; emit, per
    // column, the 8 k values as 4 dwords of k-pairs.
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = (c < 2) ? rb[2 * q].x : rb[2 * q].y;
        const uint32_t hi = (c < 2) ? rb[2 * q + 1].x : rb[2 * q + 1].y;
        o[q] = (c & 1) ? pack_hi(lo, hi) : pack_lo(lo, hi);
      }
      const int n = 4 * b_nq + c;
      *(u32x4 *)(Bs + lds_off(n, b_kb)) = o;
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][f][v] = 0.0f;

  // LDS rows of this wave's fragments.
  const int arow0 = wm * 128 + (lane & 31);
  int brow[2];
  if (DUAL) {
    brow[0] = 32 * wn + (lane & 31);
    brow[1] = 128 + 32 * wn + (lane & 31);
  } else {
    brow[0] = 64 * wn + (lane & 31);
    brow[1] = 64 * wn + 32 + (lane & 31);
  }
  const int khalf = lane >> 5;

  const int KT = (int)((K + BK - 1) / BK);
  gload(0);
  lds_store(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
    const bf16 *As = lds + cur * (2 * TILE_ELEMS);
    const bf16 *Bs = As + TILE_ELEMS;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int ch = 2 * kk + khalf;
      bf16x8 af[4], bfr[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = *(const bf16x8 *)(As + lds_off(arow0 + 32 * i, ch));
#pragma unroll
      for (int f = 0; f < 2; ++f) bfr[f] = *(const bf16x8 *)(Bs + lds_off(brow[f], ch));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int f = 0; f < 2; ++f)
          acc[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[f], acc[i][f], 0, 0, 0);
    }
    if (kt + 1 < KT) lds_store(cur ^ 1);
    __syncthreads();
  }

  // Epilogue.  32x32 accumulator layout: lane holds column (lane & 31) and rows
  // 8 (v / 4) + 4 (lane / 32) + (v % 4), v = 0..15.
  const int64_t rbase = m0 + wm * 128 + 4 * (lane >> 5);
  if constexpr (EPI == EPI_F32) {
    float *C = (float *)p.C + g * p.sC;
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int64_t col = n0 + 64 * wn + 32 * f + (lane & 31);
      if (col >= N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t row = rbase + 32 * i + 8 * (v >> 2) + (v & 3);
          if (row < M) C[row * p.ldc + col] = acc[i][f][v];
        }
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    bf16 *C = (bf16 *)p.C + g * p.sC;
    const int64_t col = n0 + 32 * wn + (lane & 31);
    if (col < N) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t row = rbase + 32 * i + 8 * (v >> 2) + (v & 3);
          if (row < M) C[row * p.ldc + col] = to_bf16(silu(acc[i][0][v]) * acc[i][1][v]);
        }
    }
  } else {
    bf16 *C = (bf16 *)p.C + g * p.sC;
    const bf16 *bias = p.bias ? (const bf16 *)p.bias + g * p.sBias : nullptr;
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int64_t col = n0 + 64 * wn + 32 * f + (lane & 31);
      if (col >= N) continue;
      const float bv = bias ? (float)bias[col] : 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t row = rbase + 32 * i + 8 * (v >> 2) + (v & 3);
          if (row < M) C[row * p.ldc + col] = to_bf16(activate<ACT>(acc[i][f][v] + bv));
        }
    }
  }
}

template <int EPI, int ACT>
hipError_t launch_t(const GemmArgs &a, hipStream_t s) {
  const int nout = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
  const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + nout - 1) / nout) * a.groups;
  if (tiles <= 0) return hipSuccess;
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_bf16_tiled_kernel<EPI, ACT>), dim3((unsigned)tiles), dim3(NTHREADS), 0,
                     s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16_tiled(const GemmArgs &a, hipStream_t s) {
  switch (a.epi) {
    case EPI_F32:
      return launch_t<EPI_F32, ACT_NONE>(a, s);
    case EPI_SWIGLU:
      return launch_t<EPI_SWIGLU, ACT_SWIGLU>(a, s);
    case EPI_ACT:
      switch (a.act) {
        case ACT_NONE:
          return launch_t<EPI_ACT, ACT_NONE>(a, s);
        case ACT_RELU:
          return launch_t<EPI_ACT, ACT_RELU>(a, s);
        case ACT_GELU_TANH:
          return launch_t<EPI_ACT, ACT_GELU_TANH>(a, s);
        case ACT_GELU_ERF:
          return launch_t<EPI_ACT, ACT_GELU_ERF>(a, s);
      }
  }
  return hipErrorInvalidValue;
}

}  // namespace tpmlp
