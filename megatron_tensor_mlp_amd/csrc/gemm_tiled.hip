// bf16 MFMA GEMM with fp32 accumulation and fused epilogues, for gfx950.
//
// Used for the column step (X * W1_i with bias + GeLU/ReLU, or the SwiGLU
// pair X * Wg_i, X * Wu_i) and the row step (Y_i * W2_i -> fp32 partial) when
// the token count is large ("Transformer math: tensor parallel", sections on
// the column- and row-parallel splits; "Tensor Parallelism Explained", 2.B).
//
// Tile: BM (256 or 128) rows x 256 accumulator columns per workgroup, NWAVE
// wave64s as (BM/128) x (NWAVE/(BM/128)), each wave owning 128 rows of
// accumulator columns as blocks of v_mfma_f32_32x32x16_bf16 accumulators.
// The default for large problems is 256 rows with 8 waves (two per SIMD), each
// 128 x 64, so the SIMD switches to the other wave whenever one waits; 4 waves
// of 128 x 128 (256 fp32 per lane, in AGPRs) exist for sweeps.  Problems with
// at most 128 tiles of 256 rows (half a 256-CU device) use 128-row tiles of
// 4 waves of 128 x 64 instead, twice as many tiles.  For
// SwiGLU the accumulator columns are 128 gate columns and the same 128 up
// columns, and each wave takes equal gate and up slices, so the gate and up
// value of an output element sit in the same lane and the epilogue is local.
//
// Data path: both operands go from HBM to LDS by buffer loads that write LDS
// directly (no register staging).  Lanes whose element lies outside the
// matrix get an offset past the buffer's range, which the hardware turns into
// zeros, so ragged tiles need no special case.
//   A (row-major [M,K], k contiguous) is kept [row][BK k]; fragments are
//     16-byte reads of 8 consecutive k.
//   B (row-major [K,N], n contiguous) is kept as it is in memory, [k][n]; the
//     MFMA wants 8 consecutive k per lane, so fragments are taken with the
//     transposing LDS read ds_read_b64_tr_b16: 16 lanes that address a 4(k) x
//     16(n) block each receive one column as 4 consecutive k.
// Both LDS tiles XOR-swizzle their 16-byte units by row so that the fragment
// reads hit distinct banks.  LDS holds NST stages of BK k each: the loads of
// step t+NST-1 are in flight while step t's MFMAs run.  Within a step every
// 16-k slice issues its MFMAs one by one, each followed by at most two memory
// instructions (the reads of the next slice's fragments, and the loads of a
// future step), in an order pinned with sched_barrier.
#include <cstdlib>

#include "device_common.hpp"
#include "kernels.h"
#include "lds_dma.hpp"

namespace tpmlp {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

constexpr int BN = 256;               // tile columns (SwiGLU: 128 gate + 128 up)
constexpr int GROUP_M = 4;            // row-tiles walked together for L2 reuse

// XOR masks on the 16-byte unit index of an LDS row.
//  A rows (2*BK bytes = BK/8 units): fragment reads touch 8 or 16 consecutive
//  rows at one logical unit; the mask spreads them over distinct banks.
template <int BK>
__device__ __forceinline__ int swz_a(int r) {
  if constexpr (BK == 64)
    return ((r >> 1) ^ (r << 2)) & 7;
  else
    return ((r >> 1) ^ (r >> 2)) & 3;
}
//  B rows (512 or 256 B): a transposing read touches 4 consecutive k rows x
//  32 or 64 bytes; rows k..k+3 get masks 0, 4, 10, 14 (distinct 64-byte
//  segments and distinct 32-byte pairs within them).
__device__ __forceinline__ int swz_b(int k) { return ((k & 3) << 2) ^ (k & 2); }

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

template <int EPI, int ACT, int BK, int NST, int NWAVE, int BM, int LAY>
__global__ __launch_bounds__(NWAVE * 64, 1) void gemm_bf16_tiled_kernel(const GemmArgs p) {
  constexpr bool DUAL = (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_SAVE);
  constexpr bool TA = (LAY == LAY_TN);  // A held as A^T [K,M]: m contiguous
  constexpr bool TB = (LAY == LAY_NT);  // B held as B^T [N,K]: k contiguous
  constexpr int NOUT = DUAL ? BN / 2 : BN;       // output columns per tile
  constexpr int KK = BK / 16;                    // 16-k MFMA slices per step
  constexpr int WMW = BM / 128;                  // waves along M (128 rows each)
  constexpr int WNW = NWAVE / WMW;               // waves along N
  constexpr int WN = BN / WNW;                   // accumulator columns per wave
  constexpr int NB = WN / 32;                    // 32-column B fragments per wave
  constexpr int NMF = 4 * NB;                    // MFMAs per slice per wave
  // A fragment is one 16-byte LDS read when its operand is k-contiguous in LDS,
  // two transposing half reads when it is m- (n-) contiguous.
  constexpr int PA = TA ? 2 : 1;                 // LDS reads per A fragment
  constexpr int PB = TB ? 1 : 2;                 // LDS reads per B fragment
  constexpr int NREAD = 4 * PA + NB * PB;        // LDS reads per slice per wave
  constexpr int A_BYTES = BM * BK * 2;           // [BM rows][BK k]
  constexpr int B_BYTES = BK * BN * 2;           // [BK k][256 cols] or 2 x [BK][128]
  constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  constexpr int AUNITS = BK / 8;                 // 16-byte units per k-contiguous row
  constexpr int AROWS_PER_LOAD = 64 / AUNITS;    // k-contiguous rows one wave-wide 1 KiB load fills
  constexpr int APITCH = TA ? 2 * BM : 2 * BK;   // bytes per A row in LDS (k rows when TA)
  constexpr int ATUNITS = BM / 8;                // 16-byte units per k row of A^T
  constexpr int AKROWS_PER_LOAD = 1024 / APITCH; // k rows of A^T one load fills
  constexpr int A_LOADS = A_BYTES / 1024 / NWAVE;  // per wave
  constexpr int BREG = DUAL ? BN / 2 : BN;       // columns per B region
  constexpr int BPITCH = BREG * 2;               // bytes per B row
  constexpr int BUNITS = BREG / 8;               // 16-byte units per B row
  constexpr int BROWS_PER_LOAD = 1024 / BPITCH;  // B rows one wave-wide load fills
  constexpr int B_LOADS = B_BYTES / 1024 / NWAVE;  // per wave
  constexpr int B_LOADS_PER_REGION = (B_BYTES / 1024) / (DUAL ? 2 : 1);
  constexpr int LPS = A_LOADS + B_LOADS;         // loads per wave per stage
  // Slot (MFMA of a slice) that issues fragment read q of the next slice:
  // R0 + q / RPS, centred in the slice.
  constexpr int RPS = (NREAD + NMF - 1) / NMF;   // reads per slot, at most
  constexpr int NRS = (NREAD + RPS - 1) / RPS;   // slots carrying reads
  constexpr int R0 = (NMF - NRS) / 2;            // first slot carrying a fragment read
  static_assert(NST >= 2 && NST <= 4, "2..4 stages");
  static_assert((BM == 128 || BM == 256) && NWAVE % WMW == 0, "tile rows");
  static_assert(NST * STAGE_BYTES <= 160 * 1024, "LDS");
  static_assert(A_LOADS >= 1 && B_LOADS >= 1 && LPS <= NMF, "load split");
  static_assert(B_LOADS_PER_REGION % B_LOADS == 0, "a wave's B loads stay in one region");

  // One LDS array per stage.
  __shared__ __attribute__((aligned(1024))) char smem0[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char smem1[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char smem2[NST > 2 ? STAGE_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) char smem3[NST > 3 ? STAGE_BYTES : 16];
  char *const stages[4] = {smem0, smem1, smem2, smem3};

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int wm = wave / WNW, wn = wave % WNW;
  const int tilesM = (int)((p.M + BM - 1) / BM), tilesN = (int)((p.N + NOUT - 1) / NOUT);
  int g, tm, tn;
  tile_coords(blockIdx.x, tilesM, tilesN, tilesM * tilesN * p.groups, g, tm, tn);

  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * NOUT;
  const bf16 *A = (const bf16 *)p.A + g * p.sA + (TA ? m0 : m0 * p.lda);
  // B offsets are taken from the matrix base: a column map may send a tile's
  // columns to separate column blocks of B.
  const bf16 *B = (const bf16 *)p.B + g * p.sB;
  const bf16 *B2 = DUAL ? (const bf16 *)p.B2 + g * p.sB2 : nullptr;

  // ---- per-lane load offsets (bytes, relative to the k-step's base) -------
  // A: load j of wave w fills rows (A_LOADS w + j) * AROWS_PER_LOAD + lane/AUNITS,
  // physical unit lane % AUNITS (logical unit = physical ^ swizzle).
  uint32_t a_off[A_LOADS];
  int a_kof[A_LOADS];
#pragma unroll
  for (int j = 0; j < A_LOADS; ++j) {
    if constexpr (!TA) {
      const int r = (A_LOADS * wave + j) * AROWS_PER_LOAD + lane / AUNITS;
      const int lu = (lane % AUNITS) ^ swz_a<BK>(r);
      a_kof[j] = 8 * lu;
      a_off[j] = (m0 + r < M) ? (uint32_t)((r * p.lda + 8 * lu) * 2) : OOB;
    } else {
      // A^T: load j fills k rows (A_LOADS w + j) * AKROWS_PER_LOAD + lane / ATUNITS
      // of BM m each; lane -> physical unit lane % ATUNITS.
      const int k = (A_LOADS * wave + j) * AKROWS_PER_LOAD + lane / ATUNITS;
      const int lu = (lane % ATUNITS) ^ swz_b(k);
      a_kof[j] = k;
      a_off[j] = (m0 + 8 * lu < M) ? (uint32_t)((k * p.lda + 8 * lu) * 2) : OOB;
    }
  }
  // B: load j of wave w is load gi = B_LOADS w + j of the tile, filling 1 KiB
  // of a B region = BROWS_PER_LOAD rows; lane -> row lane / BUNITS, unit
  // lane % BUNITS.  With SwiGLU the first half of the loads fill the gate
  // region and the second half the up region (the first and second half of
  // the waves).
  uint32_t b_off[B_LOADS];
  int b_k[B_LOADS];
  const bool b_up = DUAL && (B_LOADS * wave >= B_LOADS_PER_REGION);
#pragma unroll
  for (int j = 0; j < B_LOADS; ++j) {
    const int gi = B_LOADS * wave + j;
    const int li = gi % B_LOADS_PER_REGION;
    const int64_t ld = b_up ? p.ldb2 : p.ldb;
    if constexpr (!TB) {
      const int k = li * BROWS_PER_LOAD + lane / BUNITS;
      const int lu = (lane % BUNITS) ^ swz_b(k);
      const int64_t col = n0 + 8 * lu;  // output column of this 16-byte unit
      b_k[j] = k;
      b_off[j] = (col < N) ? (uint32_t)((k * ld + src_col(p, col)) * 2) : OOB;
    } else {
      // B^T: load j fills n rows li * AROWS_PER_LOAD + lane / AUNITS of the
      // region, BK k each, like the rows of A.
      const int r = li * AROWS_PER_LOAD + lane / AUNITS;
      const int lu = (lane % AUNITS) ^ swz_a<BK>(r);
      const int64_t col = n0 + r;  // output column of this row
      b_k[j] = 8 * lu;
      b_off[j] = (col < N) ? (uint32_t)((src_col(p, col) * ld + 8 * lu) * 2) : OOB;
    }
  }

  // This wave's loads of k-step dkt into `stage`, one at a time (q < LPS).
  // Past the last step (dkt >= KT) every lane gets an out-of-range offset: the
  // stage, which nothing reads again, is filled with zeros and no memory is
  // touched, so the pipeline needs no branch.
  struct LoadCtx {
    bool live;
    int64_t k0;
    i32x4 ra, rb;
  };
  auto load_ctx = [&](int dkt, int KT) {
    LoadCtx c;
    c.live = dkt < KT;
    c.k0 = (int64_t)(c.live ? dkt : 0) * BK;
    c.ra = rsrc(TA ? A + c.k0 * p.lda : A + c.k0);
    if constexpr (TB)  // k past ksplit comes from the second matrix (same ld)
      c.rb = rsrc(p.ksplit > 0 && c.k0 >= p.ksplit ? (const bf16 *)p.B2 + (c.k0 - p.ksplit)
                                                    : (b_up ? B2 : B) + c.k0);
    else
      c.rb = rsrc(b_up ? B2 + c.k0 * p.ldb2 : B + c.k0 * p.ldb);
    return c;
  };
  auto issue_load = [&](const LoadCtx &c, char *stage, int q) {
    if (q < A_LOADS) {
      const uint32_t off = (c.live && c.k0 + a_kof[q] < K) ? a_off[q] : OOB;
      dma16(c.ra, stage + (A_LOADS * wave + q) * 1024, off);
    } else {
      const int j = q - A_LOADS;
      const uint32_t off = (c.live && c.k0 + b_k[j] < K) ? b_off[j] : OOB;
      // regions are consecutive, so tile load gi fills bytes [gi KiB, +1 KiB)
      dma16(c.rb, stage + A_BYTES + (B_LOADS * wave + j) * 1024, off);
    }
  };

  // ---- fragment addresses ---------------------------------------------------
  // A fragment i (rows 128 wm + 32 i + lane%32) at 16-k slice kk: logical unit
  // 2 kk + lane/32.
  const int khalf = lane >> 5;
  // k-contiguous A: fragment i reads row 128 wm + 32 i + lane % 32.  A^T: the
  // transposing read, as for B below, at m columns 128 wm + 32 i + 16 (g % 2)
  // + 4 (j % 4).
  int a_row[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    a_row[i] = TA ? 128 * wm + 32 * i + 16 * ((lane >> 4) & 1) + 4 * (lane & 3)
                  : 128 * wm + 32 * i + (lane & 31);
  // B fragment f: columns cb .. cb+31 of a region; 16-lane group g = lane/16
  // reads k rows 16 kk + 8 (g/2) + 4 h + (j/4) and columns cb + 16 (g%2) + 4 (j%4).
  int b_reg_off[NB], b_col[NB];
#pragma unroll
  for (int f = 0; f < NB; ++f) {
    int region, cb;
    if (DUAL) {
      region = f / (NB / 2);
      cb = (WN / 2) * wn + 32 * (f % (NB / 2));
    } else {
      region = 0;
      cb = WN * wn + 32 * f;
    }
    b_reg_off[f] = A_BYTES + region * (BK * BPITCH);
    b_col[f] = TB ? cb + (lane & 31) : cb + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  }
  const int b_krow = 8 * (lane >> 5) + ((lane & 15) >> 2);

  bf16x8 fa[2][4], fb[2][NB];
  s16x4 fah[2][4][2];   // A^T fragments as the two transposing-read halves
  s16x4 fbh[2][NB][2];  // B fragments as the two transposing-read halves
  // Part hh of A fragment i of slice kk (the whole fragment for k-contiguous A;
  // k 0-3 or 4-7 of the lane's 8 for A^T).
  auto load_a = [&](const char *base, int kk, int i, int hh, int buf) {
    if constexpr (!TA) {
      const int r = a_row[i], u = 2 * kk + khalf;
      fa[buf][i] = *(const bf16x8 *)(base + r * (2 * BK) + ((u ^ swz_a<BK>(r)) << 4));
    } else {
      const int k = 16 * kk + 4 * hh + b_krow;
      const int c = a_row[i];
      const int off = k * APITCH + (((c >> 3) ^ swz_b(k)) << 4) + ((c & 4) << 1);
      fah[buf][i][hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(base + off));
    }
  };
  // Part hh of B fragment f of slice kk (k 0-3 or 4-7 of the lane's 8 for
  // n-contiguous B; the whole fragment for B^T).
  auto load_bh = [&](const char *base, int kk, int f, int hh, int buf) {
    if constexpr (!TB) {
      const int k = 16 * kk + 4 * hh + b_krow;
      const int c = b_col[f];
      const int off = b_reg_off[f] + k * BPITCH + (((c >> 3) ^ swz_b(k)) << 4) + ((c & 4) << 1);
      fbh[buf][f][hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(base + off));
    } else {
      const int r = b_col[f], u = 2 * kk + khalf;
      fb[buf][f] = *(const bf16x8 *)(base + b_reg_off[f] + r * (2 * BK) +
                                     ((u ^ swz_a<BK>(r)) << 4));
    }
  };
  auto join_frags = [&](int buf) {
    if constexpr (TA) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const s16x4 h0 = fah[buf][i][0], h1 = fah[buf][i][1];
        const s16x8 v = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
        fa[buf][i] = __builtin_bit_cast(bf16x8, v);
      }
    }
    if constexpr (!TB) {
#pragma unroll
      for (int f = 0; f < NB; ++f) {
        const s16x4 h0 = fbh[buf][f][0], h1 = fbh[buf][f][1];
        const s16x8 v = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
        fb[buf][f] = __builtin_bit_cast(bf16x8, v);
      }
    }
  };
  // The NREAD LDS reads of one slice, in the order its MFMAs (i-major) consume
  // them: B0 (all parts), A0, the other B fragments, then A1, A2, A3.
  auto load_piece = [&](const char *base, int kk, int buf, int q) {
    constexpr int QA0 = PB, QB1 = PB + PA, QA1 = PB + PA + (NB - 1) * PB;
    if (q < QA0)
      load_bh(base, kk, 0, q, buf);
    else if (q < QB1)
      load_a(base, kk, 0, q - QA0, buf);
    else if (q < QA1)
      load_bh(base, kk, 1 + (q - QB1) / PB, (q - QB1) % PB, buf);
    else
      load_a(base, kk, 1 + (q - QA1) / PA, (q - QA1) % PA, buf);
  };
  auto load_frags = [&](const char *base, int kk, int buf) {
#pragma unroll
    for (int q = 0; q < NREAD; ++q) load_piece(base, kk, buf, q);
    join_frags(buf);
  };

  f32x16 acc[4][NB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int f = 0; f < NB; ++f)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][f][v] = 0.0f;

  // One slice of MFMAs on buffer `buf` (i-major), interleaved slot by slot
  // with up to two memory instructions: the reads of the next slice into
  // buffer `nbuf` and, when `dctx` is given, this wave's loads of a future
  // k-step into `dstage` (slots 0..LPS-1).  sched_barrier(0) pins the order,
  // so fragment reads stay a full slice ahead of their use.
  auto slice = [&](int buf, const char *nbase, int nkk, int nbuf, const LoadCtx *dctx,
                   char *dstage) {
#pragma unroll
    for (int t = 0; t < NMF; ++t) {
      const int i = t / NB, f = t % NB;
      acc[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][f], acc[i][f], 0,
                                                          0, 0);
      if (dctx && t < LPS) issue_load(*dctx, dstage, t);
#pragma unroll
      for (int r = 0; r < RPS; ++r) {
        const int q = (t - R0) * RPS + r;
        if (t >= R0 && q < NREAD) load_piece(nbase, nkk, nbuf, q);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    join_frags(nbuf);
  };

  const int KT = (int)((K + BK - 1) / BK);
  // One k-step on stage s = kt % NST.  Step kt+NST-1 is loaded into the stage
  // read by step kt-1 (free once the barrier that ended step kt-1 passed);
  // past the last step those loads are the zero-filling kind and the
  // fragments read after the last step are never used, so nothing branches.
  auto step = [&](int kt, int s) {
    const char *cur = stages[s];
    const LoadCtx c = load_ctx(kt + NST - 1, KT);
#pragma unroll
    for (int kk = 1; kk < KK; ++kk)
      slice((kk - 1) & 1, cur, kk, kk & 1, kk == 1 ? &c : nullptr, stages[(s + NST - 1) % NST]);
    // This wave's loads of step kt+1 have landed (the NST-2 later steps may
    // still be in flight) and its fragment reads of step kt are done; the
    // barrier makes that true for every wave.
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0((NST - 2) * LPS));
    wg_barrier();
    slice((KK - 1) & 1, stages[(s + 1) % NST], 0, 0, nullptr, nullptr);
  };

#pragma unroll
  for (int s = 0; s < NST - 1; ++s) {
    const LoadCtx c = load_ctx(s, KT);
#pragma unroll
    for (int q = 0; q < LPS; ++q) issue_load(c, stages[s], q);
  }
  __builtin_amdgcn_s_waitcnt(wait_vm((NST - 2) * LPS));
  wg_barrier();
  load_frags(stages[0], 0, 0);
  int kt = 0;
  for (; kt + NST <= KT; kt += NST) {
#pragma unroll
    for (int s = 0; s < NST; ++s) step(kt + s, s);
  }
#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (kt + s < KT) step(kt + s, s);
  // No load may still be writing LDS when the workgroup releases it.
  __builtin_amdgcn_s_waitcnt(wait_vm(0));

  // ---- epilogue ---------------------------------------------------------------
  // 32x32 accumulator layout: lane holds column (lane & 31) and rows
  // 8 (v / 4) + 4 (lane / 32) + (v % 4), v = 0..15.
  const int64_t rbase = m0 + 128 * wm + 4 * (lane >> 5);
  if constexpr (EPI == EPI_F32) {
    float *C = (float *)p.C + g * p.sC;
#pragma unroll
    for (int f = 0; f < NB; ++f) {
      const int64_t col = n0 + WN * wn + 32 * f + (lane & 31);
      if (col >= N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t row = rbase + 32 * i + 8 * (v >> 2) + (v & 3);
          if (row < M) C[row * p.ldc + col] = acc[i][f][v];
        }
    }
  } else if constexpr (EPI == EPI_F32_ACC) {
    // All 16 loads of a 32-row block are issued before the first add (rows
    // past M load row M-1 and store nothing), so the block costs one memory
    // round trip instead of sixteen.
    float *C = (float *)p.C + g * p.sC;
#pragma unroll
    for (int f = 0; f < NB; ++f) {
      const int64_t col = n0 + WN * wn + 32 * f + (lane & 31);
      if (col >= N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float old[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t row = rbase + 32 * i + 8 * (v >> 2) + (v & 3);
          old[v] = C[(row < M ? row : M - 1) * p.ldc + col];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t row = rbase + 32 * i + 8 * (v >> 2) + (v & 3);
          if (row < M) C[row * p.ldc + col] = old[v] + acc[i][f][v];
        }
      }
    }
  } else if constexpr (DUAL) {
    bf16 *C = (bf16 *)p.C + g * p.sC;
    bf16 *C2 = (bf16 *)p.C2;
#pragma unroll
    for (int f = 0; f < NB / 2; ++f) {
      const int64_t col = n0 + (WN / 2) * wn + 32 * f + (lane & 31);
      if (col >= N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t row = rbase + 32 * i + 8 * (v >> 2) + (v & 3);
          if (row < M) {
            const float gv = acc[i][f][v], uv = acc[i][f + NB / 2][v];
            C[row * p.ldc + col] = to_bf16(silu(gv) * uv);
            if constexpr (EPI == EPI_SWIGLU_SAVE) {
              C2[row * p.ldc2 + col] = to_bf16(gv);
              C2[row * p.ldc2 + N + col] = to_bf16(uv);
            }
          }
        }
    }
  } else if constexpr (EPI == EPI_DACT || EPI == EPI_DSWIGLU) {
    // acc is the gradient of the activation's output; aux holds what the
    // forward kept (the pre-activation, or [gate | up]).
    bf16 *C = (bf16 *)p.C + g * p.sC;
    const bf16 *H = (const bf16 *)p.aux;
#pragma unroll
    for (int f = 0; f < NB; ++f) {
      const int64_t col = n0 + WN * wn + 32 * f + (lane & 31);
      if (col >= N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // The kept values of a 32-row block are all loaded before the first
        // use (rows past M load row M-1 and store nothing).
        constexpr int NH = EPI == EPI_DSWIGLU ? 2 : 1;
        float hv[NH][16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t row = rbase + 32 * i + 8 * (v >> 2) + (v & 3);
          const int64_t r = row < M ? row : M - 1;
#pragma unroll
          for (int q = 0; q < NH; ++q) hv[q][v] = (float)H[r * p.ldaux + q * N + col];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t row = rbase + 32 * i + 8 * (v >> 2) + (v & 3);
          if (row >= M) continue;
          const float dy = acc[i][f][v];
          if constexpr (EPI == EPI_DACT) {
            C[row * p.ldc + col] = to_bf16(dy * dactivate<ACT>(hv[0][v]));
          } else {
            const float gv = hv[0][v], uv = hv[NH - 1][v];
            C[row * p.ldc + col] = to_bf16(dy * uv * dactivate<ACT_SWIGLU>(gv));
            C[row * p.ldc + N + col] = to_bf16(dy * silu(gv));
          }
        }
      }
    }
  } else {
    bf16 *C = (bf16 *)p.C + g * p.sC;
    bf16 *C2 = (bf16 *)p.C2;
    const bf16 *bias = p.bias ? (const bf16 *)p.bias + g * p.sBias : nullptr;
#pragma unroll
    for (int f = 0; f < NB; ++f) {
      const int64_t col = n0 + WN * wn + 32 * f + (lane & 31);
      if (col >= N) continue;
      const float bv = bias ? (float)bias[src_col(p, col)] : 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t row = rbase + 32 * i + 8 * (v >> 2) + (v & 3);
          if (row < M) {
            C[row * p.ldc + col] = to_bf16(activate<ACT>(acc[i][f][v] + bv));
            if constexpr (EPI == EPI_ACT_SAVE) C2[row * p.ldc2 + col] = to_bf16(acc[i][f][v] + bv);
          }
        }
    }
  }
}

// Tile-loop configuration: (BK, stages, waves, tile rows).  Variant 1 is the
// default (256-row tiles, or 128-row tiles for small problems); 0, 2, 3 and 4
// force one configuration, for sweeps.
int tiled_variant() {
  static int v = [] {
    const char *e = getenv("TPMLP_TILED_VARIANT");
    return e ? atoi(e) : 1;
  }();
  return v;
}

template <int EPI, int ACT, int BK, int NST, int NWAVE, int BM, int LAY>
void launch_cfg(const GemmArgs &a, hipStream_t s) {
  const int nout = (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_SAVE) ? BN / 2 : BN;
  const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + nout - 1) / nout) * a.groups;
  hipLaunchKernelGGL((gemm_bf16_tiled_kernel<EPI, ACT, BK, NST, NWAVE, BM, LAY>),
                     dim3((unsigned)tiles), dim3(NWAVE * 64), 0, s, a);
}

// Tiles of 256 rows at most fill half of a 256-CU device: switch to 128-row
// tiles (4 waves of 128 x 64), twice as many, for problems that small.
constexpr int64_t SMALL_TILE_MAX = 128;

// SWEEP: the configuration variants of the forward epilogues can be forced
// for sweeps; the other instantiations take the default choice only.
template <int EPI, int ACT, int LAY, bool SWEEP>
hipError_t launch_t(const GemmArgs &a, hipStream_t s) {
  const int nout = (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_SAVE) ? BN / 2 : BN;
  const int64_t tiles = ((a.M + 255) / 256) * ((a.N + nout - 1) / nout) * a.groups;
  if (tiles <= 0) return hipSuccess;
  if (2 * tiles > 0x7fffffff) return hipErrorInvalidValue;
  int v = SWEEP ? tiled_variant() : 1;
  if (v == 1 && tiles <= SMALL_TILE_MAX) v = 4;
  if constexpr (SWEEP) {
    switch (v) {
      case 0:
        launch_cfg<EPI, ACT, 32, 4, 4, 256, LAY>(a, s);
        return hipGetLastError();
      case 2:
        launch_cfg<EPI, ACT, 64, 2, 8, 256, LAY>(a, s);
        return hipGetLastError();
      case 3:
        launch_cfg<EPI, ACT, 32, 3, 8, 256, LAY>(a, s);
        return hipGetLastError();
      default:
        break;
    }
  }
  if (v == 4)
    launch_cfg<EPI, ACT, 32, 4, 4, 128, LAY>(a, s);
  else
    launch_cfg<EPI, ACT, 32, 4, 8, 256, LAY>(a, s);
  return hipGetLastError();
}

template <int EPI, int LAY, bool SWEEP>
hipError_t launch_act(const GemmArgs &a, hipStream_t s) {
  switch (a.act) {
    case ACT_NONE:
      return launch_t<EPI, ACT_NONE, LAY, SWEEP>(a, s);
    case ACT_RELU:
      return launch_t<EPI, ACT_RELU, LAY, SWEEP>(a, s);
    case ACT_GELU_TANH:
      return launch_t<EPI, ACT_GELU_TANH, LAY, SWEEP>(a, s);
    case ACT_GELU_ERF:
      return launch_t<EPI, ACT_GELU_ERF, LAY, SWEEP>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool gemm_bf16_tiled_supported(const GemmArgs &a) {
  // Per-lane buffer offsets are 32-bit byte offsets from a tile's k-step base:
  // 256 rows of A, and 64 rows of B plus a column index below ldb, must stay
  // below 2^31 bytes; with B^T, every row of B^T the tile can reach (N of
  // them, no column map); with A^T, 64 k rows of it.
  const int64_t one = 1;
  if (a.ksplit != 0 && (a.lay != LAY_NT || a.ksplit % 32 != 0 || a.ksplit < 0 || a.ksplit >= a.K))
    return false;
  switch (a.lay) {
    case LAY_NN:
      return a.lda < (one << 21) && a.ldb < (one << 23) &&
             (a.epi != EPI_SWIGLU && a.epi != EPI_SWIGLU_SAVE ? true : a.ldb2 < (one << 23));
    case LAY_NT:
      return a.nseg == 0 && a.lda < (one << 21) && a.ldb < (one << 23) &&
             a.N * a.ldb < (one << 30) && a.epi != EPI_SWIGLU && a.epi != EPI_SWIGLU_SAVE;
    case LAY_TN:
      return a.nseg == 0 && a.lda < (one << 23) && a.ldb < (one << 23) && a.epi != EPI_SWIGLU &&
             a.epi != EPI_SWIGLU_SAVE;
  }
  return false;
}

hipError_t launch_gemm_bf16_tiled(const GemmArgs &a, hipStream_t s) {
  if (!gemm_bf16_tiled_supported(a)) return hipErrorInvalidValue;
  if (a.lay == LAY_NN) {
    switch (a.epi) {
      case EPI_F32:
        return launch_t<EPI_F32, ACT_NONE, LAY_NN, true>(a, s);
      case EPI_SWIGLU:
        return launch_t<EPI_SWIGLU, ACT_SWIGLU, LAY_NN, true>(a, s);
      case EPI_ACT:
        return launch_act<EPI_ACT, LAY_NN, true>(a, s);
      case EPI_ACT_SAVE:
        return launch_act<EPI_ACT_SAVE, LAY_NN, false>(a, s);
      case EPI_SWIGLU_SAVE:
        return launch_t<EPI_SWIGLU_SAVE, ACT_SWIGLU, LAY_NN, false>(a, s);
    }
  } else if (a.lay == LAY_NT) {
    switch (a.epi) {
      case EPI_F32:
        return launch_t<EPI_F32, ACT_NONE, LAY_NT, false>(a, s);
      case EPI_F32_ACC:
        return launch_t<EPI_F32_ACC, ACT_NONE, LAY_NT, false>(a, s);
      case EPI_DACT:
        return launch_act<EPI_DACT, LAY_NT, false>(a, s);
      case EPI_DSWIGLU:
        return launch_t<EPI_DSWIGLU, ACT_SWIGLU, LAY_NT, false>(a, s);
    }
  } else if (a.lay == LAY_TN) {
    if (a.epi == EPI_F32) return launch_t<EPI_F32, ACT_NONE, LAY_TN, false>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tpmlp
