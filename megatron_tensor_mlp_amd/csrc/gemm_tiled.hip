// bf16 MFMA GEMM with fp32 accumulation and fused epilogues, for gfx950.
//
// Used for the column step (X * W1_i with bias + GeLU/ReLU, or the SwiGLU
// pair X * Wg_i, X * Wu_i) and the row step (Y_i * W2_i -> fp32 partial) when
// the token count is large ("Transformer math: tensor parallel", sections on
// the column- and row-parallel splits; "Tensor Parallelism Explained", 2.B).
//
// Tile: 256 rows x 256 accumulator columns x 64 k per step, 256 threads (four
// wave64s as 2 x 2), each wave owning a 128 x 128 block of the tile as 4 x 4
// v_mfma_f32_32x32x16_bf16 accumulators (256 fp32 per lane, held in AGPRs).
// For SwiGLU the accumulator columns are 128 gate columns and the same 128 up
// columns; each wave takes 64 of each, so the gate and up value of an output
// element sit in the same lane and the epilogue is local.
//
// Data path: both operands go from HBM to LDS by buffer loads that write LDS
// directly (no register staging).  Lanes whose element lies outside the
// matrix get an offset past the buffer's range, which the hardware turns into
// zeros, so ragged tiles need no special case.
//   A (row-major [M,K], k contiguous) is kept [row][64 k]; fragments are
//     16-byte reads of 8 consecutive k.
//   B (row-major [K,N], n contiguous) is kept as it is in memory, [k][n]; the
//     MFMA wants 8 consecutive k per lane, so fragments are taken with the
//     transposing LDS read ds_read_b64_tr_b16: 16 lanes that address a 4(k) x
//     16(n) block each receive one column as 4 consecutive k.
// Both LDS tiles XOR-swizzle their 16-byte units by row so that the fragment
// reads hit distinct banks.  LDS holds two stages: the loads of k-step t+1 are
// in flight while step t's MFMAs run; within a step the fragments of the next
// 16-k slice are read while the current slice's MFMAs issue.
#include "device_common.hpp"
#include "kernels.h"

namespace tpmlp {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

constexpr int BM = 256, BN = 256, BK = 64, NTHREADS = 256;
constexpr int A_BYTES = BM * BK * 2;  // 32 KiB: [256 rows][64 k]
constexpr int B_BYTES = BK * BN * 2;  // 32 KiB: [64 k][256 cols] (or 2 x [64][128] for SwiGLU)
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
constexpr int GROUP_M = 4;            // row-tiles walked together for L2 reuse
constexpr uint32_t OOB = 0x80000000u; // an offset past every buffer range: reads as zero
constexpr int RSRC_WORD3 = 0x00020000;

// XOR masks on the 16-byte unit index of an LDS row.
//  A rows (128 B = 8 units): fragment reads touch 8 or 16 consecutive rows at
//  one logical unit; this mask makes them land on distinct banks.
__device__ __forceinline__ int swz_a(int r) { return ((r >> 1) ^ (r << 2)) & 7; }
//  B rows (512 or 256 B): a transposing read touches 4 consecutive k rows x
//  32 or 64 bytes; rows k..k+3 get masks 0, 4, 10, 14 (distinct 64-byte
//  segments and distinct 32-byte pairs within them).
__device__ __forceinline__ int swz_b(int k) { return ((k & 3) << 2) ^ (k & 2); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, 0x7fffffff,
                                           RSRC_WORD3);
}

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
  constexpr int NOUT = DUAL ? BN / 2 : BN;       // output columns per tile
  constexpr int BREG = DUAL ? BN / 2 : BN;       // columns per B region
  constexpr int BPITCH = BREG * 2;               // bytes per B row
  constexpr int BUNITS = BREG / 8;               // 16-byte units per B row
  constexpr int BROWS_PER_LOAD = 1024 / BPITCH;  // B rows one wave-wide load fills
  // Two stages in two distinct arrays: the DMA into one stage and the fragment
  // reads of the other are then provably disjoint, so the compiler does not
  // make the reads wait for the DMA.
  __shared__ __attribute__((aligned(1024))) char smem0[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char smem1[STAGE_BYTES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tilesM = (int)((p.M + BM - 1) / BM), tilesN = (int)((p.N + NOUT - 1) / NOUT);
  int g, tm, tn;
  tile_coords(blockIdx.x, tilesM, tilesN, tilesM * tilesN * p.groups, g, tm, tn);

  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * NOUT;
  const bf16 *A = (const bf16 *)p.A + g * p.sA + m0 * p.lda;
  const bf16 *B = (const bf16 *)p.B + g * p.sB + n0;
  const bf16 *B2 = DUAL ? (const bf16 *)p.B2 + g * p.sB2 + n0 : nullptr;

  // ---- per-lane load offsets (bytes, relative to the k-step's base) -------
  // A: wave w fills rows 64w .. 64w+63 with 8 loads of 8 rows; lane -> row
  // (lane >> 3), physical unit (lane & 7), i.e. logical unit (lane&7)^swz.
  uint32_t a_off[8];
  int a_kof[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 64 * wave + 8 * j + (lane >> 3);
    const int lu = (lane & 7) ^ swz_a(r);
    a_kof[j] = 8 * lu;
    a_off[j] = (m0 + r < M) ? (uint32_t)((r * p.lda + 8 * lu) * 2) : OOB;
  }
  // B: 32 wave-wide loads per step (8 per wave), each filling 1 KiB of a B
  // region = BROWS_PER_LOAD rows; lane -> row (lane / BUNITS), unit lane % BUNITS.
  uint32_t b_off[8];
  int b_k[8];
  bool b_up[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int gi = 8 * wave + j;  // 0..31
    const int region = DUAL ? gi / 16 : 0;
    const int li = DUAL ? gi % 16 : gi;
    const int k = li * BROWS_PER_LOAD + lane / BUNITS;
    const int lu = (lane % BUNITS) ^ swz_b(k);
    const int64_t col = 8 * lu;  // column offset from n0 within the region
    const int64_t ld = region ? p.ldb2 : p.ldb;
    b_k[j] = k;
    b_up[j] = region;
    b_off[j] = (n0 + col < N) ? (uint32_t)((k * ld + col) * 2) : OOB;
  }

  auto issue_loads = [&](int kt, char *stage) {
    const int64_t k0 = (int64_t)kt * BK;
    char *sa = stage;
    char *sb = sa + A_BYTES;
    const __amdgpu_buffer_rsrc_t ra = rsrc(A + k0);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t off = (k0 + a_kof[j] < K) ? a_off[j] : OOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t *)(sa + (64 * wave + 8 * j) * 128),
                                               16, off, 0, 0, 0);
    }
    const __amdgpu_buffer_rsrc_t rb = rsrc(B + k0 * p.ldb);
    const __amdgpu_buffer_rsrc_t rb2 = DUAL ? rsrc(B2 + k0 * p.ldb2) : rb;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t off = (k0 + b_k[j] < K) ? b_off[j] : OOB;
      const int gi = 8 * wave + j;
      char *dst = sb + gi * 1024;  // regions are consecutive, so load gi fills bytes [gi KiB, +1 KiB)
      if (DUAL && b_up[j])
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb2, (lds_void_t *)dst, 16, off, 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_t *)dst, 16, off, 0, 0, 0);
    }
  };

  // ---- fragment addresses ---------------------------------------------------
  // A fragment i (rows 128 wm + 32 i + lane%32) at 16-k slice kk: logical unit
  // 2 kk + lane/32.
  const int khalf = lane >> 5;
  int a_row[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) a_row[i] = 128 * wm + 32 * i + (lane & 31);
  // B fragment f: columns cb .. cb+31 of a region; 16-lane group g = lane/16
  // reads k rows 16 kk + 8 (g/2) + 4 h + (j/4) and columns cb + 16 (g%2) + 4 (j%4).
  int b_reg_off[4], b_col[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    int region, cb;
    if (DUAL) {
      region = f >> 1;
      cb = 64 * wn + 32 * (f & 1);
    } else {
      region = 0;
      cb = 128 * wn + 32 * f;
    }
    b_reg_off[f] = A_BYTES + region * (BK * BPITCH);
    b_col[f] = cb + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  }
  const int b_krow = 8 * (lane >> 5) + ((lane & 15) >> 2);

  bf16x8 fa[2][4], fb[2][4];
  auto load_frags = [&](const char *base, int kk, int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = a_row[i], u = 2 * kk + khalf;
      fa[buf][i] = *(const bf16x8 *)(base + r * 128 + ((u ^ swz_a(r)) << 4));
    }
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      s16x4 h[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int k = 16 * kk + 4 * hh + b_krow;
        const int c = b_col[f];
        const int off = b_reg_off[f] + k * BPITCH + (((c >> 3) ^ swz_b(k)) << 4) + ((c & 4) << 1);
        h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(base + off));
      }
      typedef short s16x8 __attribute__((ext_vector_type(8)));
      const s16x8 v = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
      fb[buf][f] = __builtin_bit_cast(bf16x8, v);
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][f][v] = 0.0f;

  auto mfmas = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int f = 0; f < 4; ++f)
        acc[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][f], acc[i][f], 0,
                                                            0, 0);
  };

  const int KT = (int)((K + BK - 1) / BK);
  // One k-step reading stage `cur` while stage `nxt` is filled for step kt+1
  // (when there is one).  The MFMAs are unconditional: only loads depend on
  // has_next, so the accumulators never flow through a branch.
  auto step = [&](const char *cur, char *nxt, int kt, bool has_next) {
    if (has_next) issue_loads(kt + 1, nxt);
    load_frags(cur, 1, 1);
    mfmas(0);
    load_frags(cur, 2, 0);
    mfmas(1);
    load_frags(cur, 3, 1);
    mfmas(0);
    // Every wave's loads of step kt+1 have landed and every wave has read its
    // last fragments of step kt before any wave moves on.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (has_next) load_frags(nxt, 0, 0);
    mfmas(1);
  };
  issue_loads(0, smem0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  load_frags(smem0, 0, 0);
  int kt = 0;
  for (; kt + 1 < KT; kt += 2) {
    step(smem0, smem1, kt, true);
    step(smem1, smem0, kt + 1, kt + 2 < KT);
  }
  if (kt < KT) step(smem0, smem1, kt, false);

  // ---- epilogue ---------------------------------------------------------------
  // 32x32 accumulator layout: lane holds column (lane & 31) and rows
  // 8 (v / 4) + 4 (lane / 32) + (v % 4), v = 0..15.
  const int64_t rbase = m0 + 128 * wm + 4 * (lane >> 5);
  if constexpr (EPI == EPI_F32) {
    float *C = (float *)p.C + g * p.sC;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int64_t col = n0 + 128 * wn + 32 * f + (lane & 31);
      if (col >= N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t row = rbase + 32 * i + 8 * (v >> 2) + (v & 3);
          if (row < M) C[row * p.ldc + col] = acc[i][f][v];
        }
    }
  } else if constexpr (DUAL) {
    bf16 *C = (bf16 *)p.C + g * p.sC;
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int64_t col = n0 + 64 * wn + 32 * f + (lane & 31);
      if (col >= N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t row = rbase + 32 * i + 8 * (v >> 2) + (v & 3);
          if (row < M) C[row * p.ldc + col] = to_bf16(silu(acc[i][f][v]) * acc[i][f + 2][v]);
        }
    }
  } else {
    bf16 *C = (bf16 *)p.C + g * p.sC;
    const bf16 *bias = p.bias ? (const bf16 *)p.bias + g * p.sBias : nullptr;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int64_t col = n0 + 128 * wn + 32 * f + (lane & 31);
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

bool gemm_bf16_tiled_supported(const GemmArgs &a) {
  // Per-lane buffer offsets are 32-bit byte offsets from a tile's k-step base:
  // 256 rows of A and 64 rows of B must stay below 2^31 bytes.
  return a.lda < (int64_t(1) << 21) && a.ldb < (int64_t(1) << 23) &&
         (a.epi != EPI_SWIGLU || a.ldb2 < (int64_t(1) << 23));
}

hipError_t launch_gemm_bf16_tiled(const GemmArgs &a, hipStream_t s) {
  if (!gemm_bf16_tiled_supported(a)) return hipErrorInvalidValue;
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
