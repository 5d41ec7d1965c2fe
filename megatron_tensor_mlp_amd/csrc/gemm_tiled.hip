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
// at most 128 tiles of 256 rows (half a 256-CU device) split K (below) or use
// 128-row tiles, twice as many: 8 waves of 128 x 32, or 4 of 128 x 64 with
// SwiGLU (whose waves need a gate and an up fragment column).  For
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
//
// Split-K.  A problem with too few tiles to fill the device (at most 120 tiles
// of 256 rows) splits K into S ranges: S workgroups per tile, each writing
// its fp32 accumulators to a partial slot of the workspace and bumping the
// tile's arrival counter; the workgroup that arrives last sums the S partials
// in k-range order (its own from registers; the order, and so the result, does
// not depend on which workgroup that is), sets the counter back to zero and
// runs the epilogue.  Partials are stored and loaded with the agent-coherent
// cache policy (sc1), as in the few-token GEMM, so no cache write-back or
// invalidate is needed between the XCDs.
#include <cstdlib>

#include "device_common.hpp"
#include "kernels.h"
#include "lds_dma.hpp"
#include "tiled_geometry.hpp"

namespace tpmlp {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

using tiled::BN;
using tiled::swz_a;
using tiled::swz_b;
using tiled::tile_coords;
static_assert(tiled::OOB_OFF == OOB, "one out-of-range offset");

// Cache-policy operand of the buffer builtins: sc1, the agent-coherent policy.
constexpr int CPOL_SC1 = 16;

// SPLIT: the k-ranges of p.splitk (> 1) meet in `ctr` (one arrival counter
// per tile, zero between launches) and `parts` (the partial slots).
template <int EPI, int ACT, int BK, int NST, int NWAVE, int BM, int LAY, bool SPLIT>
__global__ __launch_bounds__(NWAVE * 64, 1) void gemm_bf16_tiled_kernel(const GemmArgs p,
                                                                        unsigned *ctr,
                                                                        float *parts) {
  constexpr bool DUAL = (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_SAVE);
  using G = tiled::Geom<BK, NWAVE, BM, DUAL, LAY>;
  constexpr bool TA = G::TA, TB = G::TB;
  constexpr int NOUT = G::NOUT;                  // output columns per tile
  constexpr int KK = BK / 16;                    // 16-k MFMA slices per step
  constexpr int WNW = G::WNW;                    // waves along N
  constexpr int WN = G::WN;                      // accumulator columns per wave
  constexpr int NB = G::NB;                      // 32-column B fragments per wave
  constexpr int NMF = 4 * NB;                    // MFMAs per slice per wave
  // A fragment is one 16-byte LDS read when its operand is k-contiguous in LDS,
  // two transposing half reads when it is m- (n-) contiguous.
  constexpr int PA = TA ? 2 : 1;                 // LDS reads per A fragment
  constexpr int PB = TB ? 1 : 2;                 // LDS reads per B fragment
  constexpr int NREAD = 4 * PA + NB * PB;        // LDS reads per slice per wave
  constexpr int A_BYTES = G::A_BYTES, STAGE_BYTES = G::STAGE_BYTES;
  constexpr int APITCH = G::APITCH, BPITCH = G::BPITCH;
  constexpr int A_LOADS = G::A_LOADS, B_LOADS = G::B_LOADS, LPS = G::LPS;
  // Slot (MFMA of a slice) that issues fragment read q of the next slice:
  // R0 + q / RPS, centred in the slice.
  constexpr int RPS = (NREAD + NMF - 1) / NMF;   // reads per slot, at most
  constexpr int NRS = (NREAD + RPS - 1) / RPS;   // slots carrying reads
  constexpr int R0 = (NMF - NRS) / 2;            // first slot carrying a fragment read
  static_assert(NST >= 2 && NST <= 4, "2..4 stages");
  static_assert((BM == 128 || BM == 256) && NWAVE % G::WMW == 0, "tile rows");
  static_assert(NST * STAGE_BYTES <= 160 * 1024, "LDS");
  static_assert(A_LOADS >= 1 && B_LOADS >= 1 && LPS <= NMF, "load split");
  static_assert(G::B_LOADS_PER_REGION % B_LOADS == 0, "a wave's B loads stay in one region");

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
  const int total = tilesM * tilesN * p.groups;
  int tile = blockIdx.x, sidx = 0;
  if constexpr (SPLIT) tiled::split_coords(blockIdx.x, total, tile, sidx);
  int g, tm, tn;
  tile_coords(tile, tilesM, tilesN, total, g, tm, tn);

  const int64_t M = p.M, N = p.N, K = p.K;
  // This workgroup's k-range [kbeg, kend).
  int64_t kbeg = 0, kend = K;
  if constexpr (SPLIT) tiled::split_range(K, tiled::split_kc(K, p.splitk, BK), sidx, kbeg, kend);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * NOUT;
  const bf16 *A = G::template a_tile<bf16>(p, g, m0);
  const bf16 *B = G::template b_group<bf16>(p, g);
  const bf16 *B2 = G::template b2_group<bf16>(p, g);

  // ---- per-lane load offsets (bytes, relative to the k-step's base) -------
  uint32_t a_off[A_LOADS];
  int a_kof[A_LOADS];
#pragma unroll
  for (int j = 0; j < A_LOADS; ++j) G::a_load(p, m0, wave, lane, j, a_off[j], a_kof[j]);
  uint32_t b_off[B_LOADS];
  int b_k[B_LOADS];
  const bool b_up = G::b_up(wave);
#pragma unroll
  for (int j = 0; j < B_LOADS; ++j) G::b_load(p, n0, wave, lane, j, b_off[j], b_k[j]);

  // This wave's loads of k-step dkt of the range into `stage`, one at a time
  // (q < LPS).  Past the last step (dkt >= KT) every lane gets an out-of-range offset: the
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
    c.k0 = kbeg + (int64_t)(c.live ? dkt : 0) * BK;
    c.ra = rsrc(G::a_step(p, A, c.k0));
    c.rb = rsrc(G::b_step(p, B, B2, b_up, c.k0));
    return c;
  };
  auto issue_load = [&](const LoadCtx &c, char *stage, int q) {
    if (q < A_LOADS) {
      dma16(c.ra, stage + G::a_lds(wave, q), G::step_off(c.live, c.k0, a_kof[q], kend, a_off[q]));
    } else {
      const int j = q - A_LOADS;
      dma16(c.rb, stage + G::b_lds(wave, j), G::step_off(c.live, c.k0, b_k[j], kend, b_off[j]));
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

  const int KT = (int)((kend - kbeg + BK - 1) / BK);
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

  if constexpr (SPLIT) {
    // ---- split-K: publish the partial; the last arriver sums them ----------------
    __shared__ int s_last;
    const int S = p.splitk;
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
        (char *)parts + (int64_t)tile * S * G::SLOT_BYTES, 0, 0x7fffffff, RSRC_WORD3);
    const uint32_t mine = (uint32_t)(sidx * G::SLOT_BYTES);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int f = 0; f < NB; ++f)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 v = {acc[i][f][4 * q], acc[i][f][4 * q + 1], acc[i][f][4 * q + 2],
                           acc[i][f][4 * q + 3]};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), rp,
                                                 mine + G::part_off(wave, lane, i, f, q), 0,
                                                 CPOL_SC1);
        }
    // The stores have completed once vmcnt is zero; the barrier then makes
    // that true for every wave before the counter moves.
    __builtin_amdgcn_s_waitcnt(wait_vm(0));
    __syncthreads();
    if (tid == 0) {
      const unsigned prev =
          __hip_atomic_fetch_add(ctr + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = prev == (unsigned)(S - 1);
      // Nothing else touches the counter in this launch once the last
      // arriver has read it: leave it at zero for the next one.
      if (s_last) __hip_atomic_store(ctr + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!s_last) return;
    // Sum fragment by fragment, SB ranges at a time: every load of a batch is
    // issued before the first add (this workgroup's own range reads nothing:
    // an out-of-range offset), and the adds run in k-range order.
    constexpr int SB = 4;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int f = 0; f < NB; ++f) {
        f32x4 sum[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) sum[q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        for (int s0 = 0; s0 < S; s0 += SB) {
          f32x4 val[SB][4];
#pragma unroll
          for (int c = 0; c < SB; ++c) {
            const int s2 = s0 + c;
            const bool other = s2 < S && s2 != sidx;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              val[c][q] = __builtin_bit_cast(
                  f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                             rp, other ? (uint32_t)(s2 * G::SLOT_BYTES) + G::part_off(wave, lane, i, f, q)
                                       : OOB,
                             0, CPOL_SC1));
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int c = 0; c < SB; ++c) {
            const int s2 = s0 + c;
            if (s2 >= S) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const f32x4 own = {acc[i][f][4 * q], acc[i][f][4 * q + 1], acc[i][f][4 * q + 2],
                                 acc[i][f][4 * q + 3]};
              sum[q] += s2 == sidx ? own : val[c][q];
            }
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][f][4 * q + e] = sum[q][e];
      }
  }

  // ---- epilogue ---------------------------------------------------------------
  // 32x32 accumulator layout: lane holds column (lane & 31) and rows
  // 8 (v / 4) + 4 (lane / 32) + (v % 4), v = 0..15.
  const int64_t rbase = G::row_base(m0, wm, lane);
  if constexpr (EPI == EPI_F32) {
    // fp32 outputs that no later GEMM of the path reads back (the row step's
    // partial, the weight gradients) are stored with the nontemporal hint, so
    // that they do not displace operands from the caches (measured: row step
    // 207 -> 203 us, and the next step's column GEMM faster too, its operands
    // still cached).  The backward's dX, which the next launch accumulates
    // into, is stored normally.
    float *C = (float *)p.C + g * p.sC;
#pragma unroll
    for (int f = 0; f < NB; ++f) {
      const int64_t col = G::out_col(n0, wn, f, lane);
      if (col >= N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t row = G::out_row(rbase, i, v);
          if (row < M) {
            if constexpr (LAY != LAY_NT)
              __builtin_nontemporal_store(acc[i][f][v], &C[row * p.ldc + col]);
            else
              C[row * p.ldc + col] = acc[i][f][v];
          }
        }
    }
  } else if constexpr (EPI == EPI_F32_ACC) {
    // All 16 loads of a 32-row block are issued before the first add (rows
    // past M load row M-1 and store nothing), so the block costs one memory
    // round trip instead of sixteen.
    float *C = (float *)p.C + g * p.sC;
#pragma unroll
    for (int f = 0; f < NB; ++f) {
      const int64_t col = G::out_col(n0, wn, f, lane);
      if (col >= N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float old[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t row = G::out_row(rbase, i, v);
          old[v] = C[(row < M ? row : M - 1) * p.ldc + col];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t row = G::out_row(rbase, i, v);
          if (row < M) C[row * p.ldc + col] = old[v] + acc[i][f][v];
        }
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU || EPI == EPI_ACT) {
    // The activation in fp32, rounded to bf16.  Lanes 2j and 2j+1 hold
    // adjacent columns of the same rows; for each pair of rows they swap one
    // value, so that each stores two adjacent columns of one row as one 4-byte
    // word (half the store instructions, 64-byte runs per row).  N is a
    // multiple of 8, so a column pair is in range or out of range as a whole.
    bf16 *C = (bf16 *)p.C + g * p.sC;
    const bool odd = lane & 1;
    const bf16 *bias = p.bias ? (const bf16 *)p.bias + g * p.sBias : nullptr;
#pragma unroll
    for (int f = 0; f < (DUAL ? NB / 2 : NB); ++f) {
      const int64_t col = G::out_col(n0, wn, f, lane);
      if (col >= N) continue;
      const int64_t col0 = col & ~int64_t(1);
      float bv = 0.0f;
      if constexpr (EPI == EPI_ACT)
        if (bias) bv = (float)bias[src_col(p, col)];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          float y0, y1;
          if constexpr (DUAL) {
            y0 = silu_fast(acc[i][f][v]) * acc[i][f + NB / 2][v];
            y1 = silu_fast(acc[i][f][v + 1]) * acc[i][f + NB / 2][v + 1];
          } else {
            y0 = activate_fast<ACT>(acc[i][f][v] + bv);
            y1 = activate_fast<ACT>(acc[i][f][v + 1] + bv);
          }
          const uint32_t b0 = __builtin_bit_cast(uint16_t, to_bf16(y0));
          const uint32_t b1 = __builtin_bit_cast(uint16_t, to_bf16(y1));
          const uint32_t recv = swap_adjacent_lanes(odd ? b0 : b1);
          // even lane: row of v, columns (col0, col0+1); odd lane: row of v+1.
          const uint32_t word = odd ? (recv | (b1 << 16)) : (b0 | (recv << 16));
          const int64_t row = G::out_row(rbase, i, v) + (odd ? 1 : 0);
          if (row < M) *(uint32_t *)(C + row * p.ldc + col0) = word;
        }
    }
  } else if constexpr (DUAL) {
    bf16 *C = (bf16 *)p.C + g * p.sC;
    bf16 *C2 = (bf16 *)p.C2;
#pragma unroll
    for (int f = 0; f < NB / 2; ++f) {
      const int64_t col = G::out_col(n0, wn, f, lane);
      if (col >= N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t row = G::out_row(rbase, i, v);
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
      const int64_t col = G::out_col(n0, wn, f, lane);
      if (col >= N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // The kept values of a 32-row block are all loaded before the first
        // use (rows past M load row M-1 and store nothing).
        constexpr int NH = EPI == EPI_DSWIGLU ? 2 : 1;
        float hv[NH][16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t row = G::out_row(rbase, i, v);
          const int64_t r = row < M ? row : M - 1;
#pragma unroll
          for (int q = 0; q < NH; ++q) hv[q][v] = (float)H[r * p.ldaux + q * N + col];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t row = G::out_row(rbase, i, v);
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
      const int64_t col = G::out_col(n0, wn, f, lane);
      if (col >= N) continue;
      const float bv = bias ? (float)bias[src_col(p, col)] : 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t row = G::out_row(rbase, i, v);
          if (row < M) {
            C[row * p.ldc + col] = to_bf16(activate<ACT>(acc[i][f][v] + bv));
            if constexpr (EPI == EPI_ACT_SAVE) C2[row * p.ldc2 + col] = to_bf16(acc[i][f][v] + bv);
          }
        }
    }
  }
}

// Tile-loop configuration: (BK, stages, waves, tile rows).  Variant 1 is the
// default (256-row tiles, or 128-row tiles for small problems); 0, 2, 3, 4 and 5
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
  hipLaunchKernelGGL((gemm_bf16_tiled_kernel<EPI, ACT, BK, NST, NWAVE, BM, LAY, false>),
                     dim3((unsigned)tiles), dim3(NWAVE * 64), 0, s, a, (unsigned *)nullptr,
                     (float *)nullptr);
}

// Split-K launch: 256-row tiles of 8 waves, a.splitk > 1 k-ranges each.
template <int EPI, int ACT, int LAY>
void launch_split(const GemmArgs &a, void *ws, hipStream_t s) {
  const int nout = (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_SAVE) ? BN / 2 : BN;
  const int64_t tiles = ((a.M + 255) / 256) * ((a.N + nout - 1) / nout) * a.groups;
  hipLaunchKernelGGL((gemm_bf16_tiled_kernel<EPI, ACT, 32, 4, 8, 256, LAY, true>),
                     dim3((unsigned)(tiles * a.splitk)), dim3(8 * 64), 0, s, a, (unsigned *)ws,
                     (float *)((char *)ws + kWsCounterBytes));
}

// Tiles of 256 rows at most fill half of a 256-CU device: switch to 128-row
// tiles, twice as many, for problems that small (and not split).
constexpr int64_t SMALL_TILE_MAX = 128;

// Split-K plan for problems of t <= 120 tiles of 256 rows (measured on the
// Llama-70B shapes at T = 256 .. 4096):
//  - the last arriver reads S - 1 partials of 256 KiB from the coherent
//    level at a few microseconds each, so S stays at 4 or below unless the
//    tiles are very few (t <= 20: up to 8);
//  - more than ~240 busy CUs buy little (the chip is at its power limit), so
//    t * S stays at or below 240, and at t > 120 nothing is split;
//  - S = 2 already beats the 128-row configuration (8 waves per CU instead
//    of 4, at the same workgroup count);
//  - every k-range is at least 768 long.
constexpr int SPLIT_WGS = 240;
constexpr int SPLIT_MAX = 8;
constexpr int SPLIT_MAX_MANY = 4;
constexpr int64_t SPLIT_FEW_TILES = 20;
constexpr int64_t SPLIT_MIN_K = 768;

bool split_eligible(const GemmArgs &a) {
  return a.lay == LAY_NN && a.ksplit == 0 &&
         (a.epi == EPI_F32 || a.epi == EPI_ACT || a.epi == EPI_SWIGLU);
}
int64_t tiles256(const GemmArgs &a) {
  const int nout = (a.epi == EPI_SWIGLU || a.epi == EPI_SWIGLU_SAVE) ? BN / 2 : BN;
  return ((a.M + 255) / 256) * ((a.N + nout - 1) / nout) * a.groups;
}
// TPMLP_TILED_SPLIT (read once) forces the k-ranges of every eligible GEMM
// (1: none), for sweeps.
int forced_split() {
  static int v = [] {
    const char *e = getenv("TPMLP_TILED_SPLIT");
    return e ? atoi(e) : 0;
  }();
  return v;
}

// The k-ranges a launch takes when S are asked for: ceil(K / kc) (S or fewer).
int effective_split(int64_t K, int S) {
  if (S <= 1 || K <= 0) return 1;
  const int64_t kc = tiled::split_kc(K, S, 32);
  return (int)((K + kc - 1) / kc);
}

// SWEEP: the configuration variants of the forward epilogues can be forced
// for sweeps; the other instantiations take the default choice only.
template <int EPI, int ACT, int LAY, bool SWEEP>
hipError_t launch_t(const GemmArgs &a, void *ws, hipStream_t s) {
  const int nout = (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_SAVE) ? BN / 2 : BN;
  const int64_t tiles = ((a.M + 255) / 256) * ((a.N + nout - 1) / nout) * a.groups;
  if (tiles <= 0) return hipSuccess;
  if (2 * tiles > 0x7fffffff) return hipErrorInvalidValue;
  if constexpr (SWEEP && LAY == LAY_NN && (EPI == EPI_F32 || EPI == EPI_ACT || EPI == EPI_SWIGLU)) {
    const int S = tiled_splitk(a);
    if (S > 1) {
      if (!ws) return hipErrorInvalidValue;
      GemmArgs b = a;
      b.splitk = S;
      launch_split<EPI, ACT, LAY>(b, ws, s);
      return hipGetLastError();
    }
  }
  constexpr bool DUAL = (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_SAVE);
  int v = SWEEP ? tiled_variant() : 1;
  // Small problems: 128-row tiles; 8 waves of 128 x 32 where the epilogue
  // needs no gate/up pair (measured on the GPT shard's 128 tiles: 4-6 %
  // faster than 4 waves of 128 x 64), else 4 waves.
  if (v == 1 && tiles <= SMALL_TILE_MAX) v = (SWEEP && !DUAL) ? 5 : 4;
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
      case 5:  // 128-row tiles of 8 waves of 128 x 32 (one fragment column: not SwiGLU)
        if constexpr (!DUAL) {
          launch_cfg<EPI, ACT, 32, 4, 8, 128, LAY>(a, s);
          return hipGetLastError();
        }
        break;
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
hipError_t launch_act(const GemmArgs &a, void *ws, hipStream_t s) {
  switch (a.act) {
    case ACT_NONE:
      return launch_t<EPI, ACT_NONE, LAY, SWEEP>(a, ws, s);
    case ACT_RELU:
      return launch_t<EPI, ACT_RELU, LAY, SWEEP>(a, ws, s);
    case ACT_GELU_TANH:
      return launch_t<EPI, ACT_GELU_TANH, LAY, SWEEP>(a, ws, s);
    case ACT_GELU_ERF:
      return launch_t<EPI, ACT_GELU_ERF, LAY, SWEEP>(a, ws, s);
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

int tiled_splitk(const GemmArgs &a) {
  if (!split_eligible(a) || a.splitk == 1 || a.M <= 0 || a.N <= 0) return 1;
  const int64_t t = tiles256(a);
  if (t > kWsMaxBlocks) return 1;  // one arrival counter per tile
  const int ask = a.splitk > 1 ? a.splitk : forced_split();
  if (ask >= 1) return effective_split(a.K, ask < SPLIT_MAX ? ask : SPLIT_MAX);
  if (t <= 0 || 2 * t > SPLIT_WGS) return 1;
  int64_t S = SPLIT_WGS / t;
  const int64_t cap = t <= SPLIT_FEW_TILES ? SPLIT_MAX : SPLIT_MAX_MANY;
  if (S > cap) S = cap;
  if (S > a.K / SPLIT_MIN_K) S = a.K / SPLIT_MIN_K;
  return S >= 2 ? effective_split(a.K, (int)S) : 1;
}

size_t tiled_workspace_bytes(const GemmArgs &a) {
  const int S = tiled_splitk(a);
  if (S <= 1) return 0;
  using G = tiled::Geom<32, 8, 256, false, LAY_NN>;
  static_assert(tiled::Geom<32, 8, 256, true, LAY_NN>::SLOT_BYTES == G::SLOT_BYTES, "slot");
  return kWsCounterBytes + (size_t)tiles256(a) * S * G::SLOT_BYTES;
}

hipError_t launch_gemm_bf16_tiled(const GemmArgs &a, void *ws, hipStream_t s) {
  if (!gemm_bf16_tiled_supported(a)) return hipErrorInvalidValue;
  if (a.lay == LAY_NN) {
    switch (a.epi) {
      case EPI_F32:
        return launch_t<EPI_F32, ACT_NONE, LAY_NN, true>(a, ws, s);
      case EPI_SWIGLU:
        return launch_t<EPI_SWIGLU, ACT_SWIGLU, LAY_NN, true>(a, ws, s);
      case EPI_ACT:
        return launch_act<EPI_ACT, LAY_NN, true>(a, ws, s);
      case EPI_ACT_SAVE:
        return launch_act<EPI_ACT_SAVE, LAY_NN, false>(a, ws, s);
      case EPI_SWIGLU_SAVE:
        return launch_t<EPI_SWIGLU_SAVE, ACT_SWIGLU, LAY_NN, false>(a, ws, s);
    }
  } else if (a.lay == LAY_NT) {
    switch (a.epi) {
      case EPI_F32:
        return launch_t<EPI_F32, ACT_NONE, LAY_NT, false>(a, ws, s);
      case EPI_F32_ACC:
        return launch_t<EPI_F32_ACC, ACT_NONE, LAY_NT, false>(a, ws, s);
      case EPI_DACT:
        return launch_act<EPI_DACT, LAY_NT, false>(a, ws, s);
      case EPI_DSWIGLU:
        return launch_t<EPI_DSWIGLU, ACT_SWIGLU, LAY_NT, false>(a, ws, s);
    }
  } else if (a.lay == LAY_TN) {
    if (a.epi == EPI_F32) return launch_t<EPI_F32, ACT_NONE, LAY_TN, false>(a, ws, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tpmlp
