// Few-token (T <= 64) bf16 GEMM for gfx950: the decode regime, where each
// shard's weights are read once per step and HBM bandwidth sets the time.
// ("What is Tensor Parallelism?", Llama 3.1 70B worked example: a decode token
// is tiny next to the 3584-column weight shard every GPU streams.)
//
// Weight streaming.  A workgroup owns 128 columns of one weight matrix and one
// of S contiguous k-ranges.  The range is streamed in stages of BK k rows by
// buffer loads that write LDS directly, a few stages deep (about 32 KiB in
// flight per CU measured best), without holding a register; the token rows
// (padded to 16, 32 or 64 with zeros) come along in the same stages.  Each
// weight row is read in runs of 256 contiguous bytes, with the nontemporal
// hint (weights are read once per step; the token rows, read by every
// workgroup, stay cached).  Each of the 8 waves
// owns a 16-column block: per 32-k slice it takes its weight fragment with the
// transposing LDS read ds_read_b64_tr_b16 (the weights stay [k][n] as stored)
// and multiplies it with v_mfma_f32_16x16x32_bf16.  LDS rows are XOR-swizzled
// in 16-byte units so that the fragment reads hit distinct banks.
//
// SwiGLU runs as one GEMM over both matrices: a column block's gate and up
// halves are separate workgroups (the grid walks the gate blocks, then the up
// blocks, of each k-range), and they meet in the split-K reduction, which
// applies SiLU(gate) * up.  Each workgroup thus streams a single matrix,
// which HBM serves faster than two interleaved ones.
//
// Split-K.  Every workgroup of a block writes its fp32 partial to the
// workspace and bumps the block's arrival counter (unless it is the block's
// only one); the workgroup that arrives last sums the partials in k-range
// order (so the result does not depend on which one that is), applies the
// epilogue and sets the counter back to zero.  Partials are stored and loaded
// 16 bytes per lane with the cache policy of agent-scope atomics (sc1), which
// stays coherent across the XCDs without flushing or invalidating the L2
// caches (a release or acquire fence at agent scope would do both, at a cost
// of several microseconds per workgroup); the last arriver issues all loads
// of a batch before its first add, so the reduction costs about one memory
// round trip.
#include <cstdlib>

#include "decode_geometry.hpp"
#include "device_common.hpp"
#include "kernels.h"
#include "lds_dma.hpp"

namespace tpmlp {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

// Cache-policy operand of the buffer builtins: sc1, the agent-coherent policy.
constexpr int CPOL_SC1 = 16;

using decode::Geo;
using decode::NWAVE;
using decode::RC;
using decode::RP;
using decode::swz_w;
using decode::swz_x;
static_assert(decode::OOB_OFF == OOB, "one out-of-range offset");
// The split aims at about one workgroup per CU of a 256-CU device: the
// streaming rate of a CU is what one workgroup reaches, so a CU given two
// takes twice as long (measured: 448 or 504 workgroups are slower than 224).
// TPMLP_DECODE_TARGET overrides it, for sweeps (read once).
int target_wgs() {
  static int v = [] {
    const char *e = getenv("TPMLP_DECODE_TARGET");
    const int t = e ? atoi(e) : 0;
    return t > 0 ? t : 256;
  }();
  return v;
}
constexpr int MIN_STAGES = 4;   // fewest k-steps a workgroup streams
// The workspace starts with a counter area of fixed size, so that calls with
// different plans (or other entry points) reusing one workspace never take
// partials for counters: counters of any plan lie below CTR_AREA and partials
// above it.
constexpr int64_t MAX_BLOCKS = kWsMaxBlocks;  // column blocks per call
constexpr size_t CTR_AREA = kWsCounterBytes;

struct DecodePlan {
  int64_t nblk;  // output column blocks
  int nmat;      // matrices per block (2 with SwiGLU)
  int64_t S;     // k-ranges (split-K factor)
  int64_t kc;    // k per range (multiple of bk)
  int mb;        // 16-row token blocks (1, 2 or 4)
  int bk;        // k rows per stage
};

int split_override() {
  static int v = [] {
    const char *e = getenv("TPMLP_DECODE_SPLIT");
    return e ? atoi(e) : 0;
  }();
  return v;
}

// Configurations (measured on the Llama-70B TP=8 decode shard): 32-row stages
// 4 deep; for 64 tokens, whose token rows take a third of a 32-row stage,
// 64-row stages 3 deep.
DecodePlan make_plan(const GemmArgs &a) {
  DecodePlan pl;
  pl.nmat = a.epi == EPI_SWIGLU ? 2 : 1;
  pl.mb = a.M <= 16 ? 1 : (a.M <= 32 ? 2 : 4);
  pl.bk = pl.mb == 4 ? 64 : 32;
  pl.nblk = (a.N + RC - 1) / RC;
  const int64_t steps = (a.K + pl.bk - 1) / pl.bk;
  int64_t S = target_wgs() / (pl.nblk * pl.nmat);
  int64_t smax = steps / MIN_STAGES;
  if (smax < 1) smax = 1;
  if (S > smax) S = smax;
  if (S < 1) S = 1;
  if (split_override() > 0) S = split_override() < 4096 ? split_override() : 4096;
  const int64_t per = (steps + S - 1) / S;
  pl.kc = per * pl.bk;
  pl.S = (a.K + pl.kc - 1) / pl.kc;
  return pl;
}


size_t plan_ws_bytes(const DecodePlan &pl) {
  const int64_t parts = pl.S * pl.nmat;  // workgroups per block
  if (parts <= 1) return 0;
  return CTR_AREA +
         (size_t)pl.nblk * parts * (NWAVE * pl.mb * 256) * sizeof(float);
}

// Output of one 16-column block.  Lane layout of a 16x16 accumulator block:
// column lane % 16, rows 4 (lane / 16) + v.  With SwiGLU `up` holds the
// matching up-projection sums.
template <int EPI, int ACT, int MB>
__device__ __forceinline__ void store_out(const GemmArgs &p, int64_t col, int lane,
                                          const f32x4 (&acc)[MB], const f32x4 (&up)[MB]) {
  if (col >= p.N) return;
  float bv = 0.0f;
  if constexpr (EPI == EPI_ACT)
    if (p.bias) bv = (float)((const bf16 *)p.bias)[src_col(p, col)];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t row = decode::out_row(m, lane, v);
      if (row >= p.M) continue;
      if constexpr (EPI == EPI_SWIGLU)
        ((bf16 *)p.C)[row * p.ldc + col] = to_bf16(silu(acc[m][v]) * up[m][v]);
      else if constexpr (EPI == EPI_F32)
        ((float *)p.C)[row * p.ldc + col] = acc[m][v];
      else
        ((bf16 *)p.C)[row * p.ldc + col] = to_bf16(activate<ACT>(acc[m][v] + bv));
    }
}

template <int EPI, int ACT, int MB, int BK, int NST>
__global__ __launch_bounds__(NWAVE * 64) void gemm_bf16_decode_kernel(const GemmArgs p,
                                                                      int64_t nblk, int64_t S,
                                                                      int64_t kc, unsigned *ctr,
                                                                      float *parts) {
  using G = Geo<MB, BK, NST>;
  constexpr bool DUAL = (EPI == EPI_SWIGLU);
  constexpr int NMAT = DUAL ? 2 : 1;
  __shared__ __attribute__((aligned(1024))) char smem[NST * G::SB];
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int64_t blk, s;
  bool up;
  decode::wg_coords(blockIdx.x, NMAT, nblk, blk, s, up);
  const bf16 *W = (const bf16 *)(up ? p.B2 : p.B);
  const int64_t ldw = up ? p.ldb2 : p.ldb;
  const int64_t M = p.M;
  int64_t kbeg, kend;
  decode::k_range(s, kc, p.K, kbeg, kend);
  const int nstages = (int)((kend - kbeg + BK - 1) / BK);
  const int64_t n0 = blk * RC;  // first column of the block

  // ---- per-lane load offsets, relative to a stage's k base -----------------
  uint32_t w_off[G::WL];
  int w_row[G::WL];
#pragma unroll
  for (int j = 0; j < G::WL; ++j) G::w_load(p, ldw, n0, wave, lane, j, w_off[j], w_row[j]);
  uint32_t x_off[G::XL];
  int x_k[G::XL];
#pragma unroll
  for (int j = 0; j < G::XL; ++j) G::x_load(p, wave, lane, j, x_off[j], x_k[j]);
  const bf16 *X = (const bf16 *)p.A;

  // Loads of stage t into its buffer; past the last stage every lane gets an
  // out-of-range offset, so nothing is read and no branch is needed.
  auto issue_stage = [&](int t) {
    char *st = smem + (t % NST) * G::SB;
    const bool live = t < nstages;
    const int64_t k0 = kbeg + (int64_t)(live ? t : 0) * BK;
    const i32x4 rw = rsrc(W + k0 * ldw);
    const i32x4 rx = rsrc(X + k0);
#pragma unroll
    for (int j = 0; j < G::WL; ++j)
      dma16_nt(rw, st + G::w_lds(wave, j), G::stage_off(live, k0, w_row[j], kend, w_off[j]));
#pragma unroll
    for (int j = 0; j < G::XL; ++j) {
      const uint32_t off = G::stage_off(live, k0, x_k[j], kend, x_off[j]);
      char *dst = st + G::x_lds(wave, j);
      if constexpr (G::XLB == 1024)
        dma16(rx, dst, off);
      else if (G::x_lane(lane))
        dma4(rx, dst, off);
    }
  };

  // ---- fragment addresses ------------------------------------------------------
  // Block of wave w (columns 16 w ..) at slice kk, half h: the 16-lane group g
  // reads rows 32 kk + 8 g + 4 h + (lane % 16) / 4 at columns 16 w + 4 (lane % 4);
  // the transposing read hands lane i column 16 w + i of those 4 rows.
  int w_rd[G::KS][2];
#pragma unroll
  for (int kk = 0; kk < G::KS; ++kk)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int j = lane & 15;
      const int r = 32 * kk + 8 * (lane >> 4) + 4 * h + (j >> 2);
      const int c = 16 * wave + 4 * (j & 3);
      w_rd[kk][h] = r * RP + (((c >> 3) ^ swz_w(r)) << 4) + ((c & 4) << 1);
    }
  // Token fragment of block m, slice kk: lane reads row 16 m + lane % 16,
  // logical unit 4 kk + lane / 16 (8 consecutive k).
  int x_rd[MB][G::KS];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int kk = 0; kk < G::KS; ++kk) {
      const int r = 16 * m + (lane & 15);
      const int lu = 4 * kk + (lane >> 4);
      x_rd[m][kk] = G::WB + r * G::XP + ((lu ^ swz_x<G::XP>(r)) << 4);
    }

  f32x4 acc[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) acc[m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // ---- the stream ----------------------------------------------------------------
#pragma unroll
  for (int t = 0; t < NST - 1; ++t) issue_stage(t);
  for (int t = 0; t < nstages; ++t) {
    // This wave's loads of stage t have landed once at most NST-2 later
    // stages' are pending; after the barrier every wave's have, and every wave
    // is done reading stage t-1, whose buffer the next loads reuse.
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0((NST - 2) * G::LPS));
    wg_barrier();
    issue_stage(t + NST - 1);
    const char *st = smem + (t % NST) * G::SB;
#pragma unroll
    for (int kk = 0; kk < G::KS; ++kk) {
      bf16x8 xa[MB];
#pragma unroll
      for (int m = 0; m < MB; ++m) xa[m] = *(const bf16x8 *)(st + x_rd[m][kk]);
      const s16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(st + w_rd[kk][0]));
      const s16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(st + w_rd[kk][1]));
      const s16x8 bv = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
#pragma unroll
      for (int m = 0; m < MB; ++m)
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[m], __builtin_bit_cast(bf16x8, bv),
                                                         acc[m], 0, 0, 0);
    }
  }
  // The loads issued past the last stage read nothing but still write LDS:
  // none may be pending when the workgroup ends.
  __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));

  const int64_t col = decode::out_col(n0, wave, lane);
  const int64_t nparts = NMAT * S;  // workgroups of this column block
  if (nparts == 1) {
    store_out<EPI, ACT, MB>(p, col, lane, acc, acc);
    return;
  }

  // ---- split-K: publish the partial; the last arriver reduces --------------------
  // Partials are written and read with the sc1 cache policy (what agent-scope
  // atomics use), which the hardware keeps coherent across the XCDs' L2 caches
  // without a cache write-back or invalidate; a wave's stores have completed
  // once vmcnt reaches zero, before the barrier that precedes the counter
  // update.  Slots of a block: the S gate (or only) partials in k-range order,
  // then the S up partials.  A slot holds [wave][m][lane] 16-byte groups (lane
  // accumulator block m: rows 16 m + 4 (lane / 16) + 0..3 of column lane % 16);
  // groups with no token row below M (padding) are neither written nor read:
  // their lanes get an offset past the buffer range, which the hardware drops
  // (stores) or reads as zero (loads).
  const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
      parts + blk * G::block_floats(nparts), 0, 0x7fffffff, RSRC_WORD3);
  uint32_t goff[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) goff[m] = G::group_off(M, wave, lane, m);
  {
    const uint32_t mine = G::slot_off(up ? 1 : 0, S, s);
#pragma unroll
    for (int m = 0; m < MB; ++m)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, acc[m]), rp,
                                             goff[m] == OOB ? OOB : goff[m] + mine, 0, CPOL_SC1);
  }
  __builtin_amdgcn_s_waitcnt(wait_vm(0));
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(ctr + blk, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (unsigned)(nparts - 1);
  }
  __syncthreads();
  if (!s_last) return;

  // The last arriver loads RCH k-ranges of each matrix at a time, every load
  // of a batch issued before any is added (ranges past S read nothing and add
  // nothing), and sums gate and up each in k-range order.  Which sum a slot
  // feeds is fixed at compile time: a run-time choice would put a branch, and
  // so a wait, between the loads.  RCH is sized so that the batch stays within
  // 64 VGPRs, which keeps the kernel within 128 (two workgroups per CU).
  constexpr int RCH0 = 64 / (NMAT * MB * 4);
  constexpr int RCH = RCH0 < 2 ? 2 : (RCH0 > 32 ? 32 : RCH0);
  f32x4 sum[NMAT][MB];
#pragma unroll
  for (int q = 0; q < NMAT; ++q)
#pragma unroll
    for (int m = 0; m < MB; ++m) sum[q][m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int64_t s2 = 0; s2 < S; s2 += RCH) {
    f32x4 val[NMAT][RCH][MB];
#pragma unroll
    for (int q = 0; q < NMAT; ++q)
#pragma unroll
      for (int c = 0; c < RCH; ++c) {
#pragma unroll
        for (int m = 0; m < MB; ++m) val[q][c][m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if (s2 + c < S) {  // uniform: a scalar branch, no wait
          const uint32_t slot = G::slot_off(q, S, s2 + c);
#pragma unroll
          for (int m = 0; m < MB; ++m)
            val[q][c][m] = __builtin_bit_cast(
                f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                           rp, goff[m] != OOB ? goff[m] + slot : OOB, 0, CPOL_SC1));
        }
      }
    // Keep the scheduler from interleaving the adds with the loads (it would,
    // to save registers, and each add waits for its load).
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < RCH; ++c)
      if (s2 + c < S) {
#pragma unroll
        for (int q = 0; q < NMAT; ++q)
#pragma unroll
          for (int m = 0; m < MB; ++m) sum[q][m] += val[q][c][m];
      }
  }
  if (tid == 0) __hip_atomic_store(ctr + blk, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  store_out<EPI, ACT, MB>(p, col, lane, sum[0], sum[NMAT - 1]);
}

template <int EPI, int ACT, int MB, int BK, int NST>
hipError_t launch_plan(const GemmArgs &a, const DecodePlan &pl, void *ws, hipStream_t st) {
  unsigned *ctr = nullptr;
  float *parts = nullptr;
  if (pl.S * pl.nmat > 1) {
    ctr = (unsigned *)ws;
    parts = (float *)((char *)ws + CTR_AREA);
  }
  hipLaunchKernelGGL((gemm_bf16_decode_kernel<EPI, ACT, MB, BK, NST>),
                     dim3((unsigned)(pl.nblk * pl.nmat * pl.S)), dim3(NWAVE * 64), 0, st, a,
                     pl.nblk, pl.S, pl.kc, ctr, parts);
  return hipGetLastError();
}

// The configurations make_plan chooses.
template <int EPI, int ACT>
hipError_t launch_mb(const GemmArgs &a, const DecodePlan &pl, void *ws, hipStream_t st) {
  switch (pl.mb) {
    case 1:
      return launch_plan<EPI, ACT, 1, 32, 4>(a, pl, ws, st);
    case 2:
      return launch_plan<EPI, ACT, 2, 32, 4>(a, pl, ws, st);
    default:
      return launch_plan<EPI, ACT, 4, 64, 3>(a, pl, ws, st);
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

bool gemm_bf16_decode_supported(const GemmArgs &a) {
  // Per-lane buffer offsets are 32-bit byte offsets from a stage's k base:
  // 64 weight rows and 64 token rows must stay below 2^31 bytes.  The column
  // blocks of one call must fit the counter area.
  return a.lay == LAY_NN && (a.epi == EPI_ACT || a.epi == EPI_SWIGLU || a.epi == EPI_F32) &&
         a.M >= 1 && a.M <= 64 && a.lda < (int64_t(1) << 23) && a.ldb < (int64_t(1) << 23) &&
         (a.epi != EPI_SWIGLU || a.ldb2 < (int64_t(1) << 23)) && (a.N + RC - 1) / RC <= MAX_BLOCKS;
}

hipError_t launch_gemm_bf16_decode(const GemmArgs &a, void *ws, hipStream_t st) {
  if (!gemm_bf16_decode_supported(a)) return hipErrorInvalidValue;
  // Groups run one after another on the stream; they share the workspace,
  // whose counters every launch leaves at zero.
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
