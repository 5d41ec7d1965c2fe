// Few-token (T <= 64) bf16 GEMM for gfx950: the decode regime, where each
// shard's weights are read once per step and HBM bandwidth sets the time.
// ("What is Tensor Parallelism?", Llama 3.1 70B worked example: a decode token
// is tiny next to the 3584-column weight shard every GPU streams.)
//
// Weight streaming.  A workgroup owns a block of weight columns in each of its
// regions (one matrix; with SwiGLU two, gate and up, over the same columns)
// and one of S contiguous k-ranges.  The range is streamed in stages of 64 k
// rows by buffer loads that write LDS directly, three stages deep, without
// holding a register; the token rows (padded to 16, 32 or 64 with zeros) come
// along in the same stages.  Each region row is 256 or 512 contiguous bytes of
// a weight row (HBM serves such runs at close to its streaming rate; 128-byte
// runs lose about a tenth).  Each of the 8 waves owns 16-column blocks of
// every region: per 32-k slice it takes its weight fragments with the
// transposing LDS read ds_read_b64_tr_b16 (the weights stay [k][n] as stored)
// and multiplies them with v_mfma_f32_16x16x32_bf16.  LDS rows are
// XOR-swizzled in 16-byte units so that the fragment reads hit distinct banks.
//
// Split-K.  With S > 1 every workgroup writes its fp32 partial to the
// workspace and bumps the arrival counter of its column block; the workgroup
// that arrives last sums the S partials in k-range order (so the result does
// not depend on which one that is), applies the epilogue and sets the counter
// back to zero.  Partials are stored and loaded as agent-scope atomics, which
// stay coherent across the XCDs without flushing or invalidating the L2
// caches (a release or acquire fence at agent scope would do both, at a cost
// of several microseconds per workgroup).
#include <cstdlib>

#include "device_common.hpp"
#include "kernels.h"
#include "lds_dma.hpp"

namespace tpmlp {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

constexpr int NWAVE = 8;
constexpr int NST = 3;         // stages in LDS (two in flight while one is used)
// The split aims at about one workgroup per CU of a 256-CU device.
constexpr int TARGET_WGS = 256;
constexpr int MIN_STAGES = 4;  // fewest stages a workgroup streams
constexpr int CTR_BYTES = 256; // counter area rounding

// Block geometry.  A workgroup has NW waves; a stage holds BK k rows, in NR
// regions (2 with SwiGLU: gate and up, over the same columns).  Each wave owns
// one 16-column block: normally the same block of every region (RC = 16 NW
// columns, and a SwiGLU wave holds matching gate and up sums in the same
// lanes); in the HALF layout (SwiGLU only) the first half of the waves own the
// gate blocks and the second half the up blocks (RC = 8 NW columns).
template <int EPI, bool HALF, int MB, int BK, int NW>
struct Geo {
  static constexpr int NR = EPI == EPI_SWIGLU ? 2 : 1;
  static_assert(!HALF || NR == 2, "the HALF layout pairs gate and up waves");
  static constexpr int KS = BK / 32;             // 32-k MFMA slices per stage
  static constexpr int RC = HALF ? 8 * NW : 16 * NW;  // columns per region
  static constexpr int RP = RC * 2;              // bytes per region row
  static constexpr int RPL = 1024 / RP;          // region rows per 1 KiB load
  static constexpr int RB = BK * RP;             // bytes per region per stage
  static constexpr int WB = NR * RB;             // weight bytes per stage
  static constexpr int XP = BK * 2;              // bytes per token row
  static constexpr int XB = 16 * MB * XP;        // token bytes per stage
  static constexpr int SB = WB + XB;             // stage bytes
  static constexpr int NBT = HALF ? 1 : NR;      // 16-column blocks per wave
  static constexpr int WL = WB / 1024 / NW;      // 1 KiB weight loads per wave per stage
  // Token rows: XB / NW bytes per wave, in 1 KiB loads (16 B per lane) when
  // there are at least that many, else in 256 B loads (4 B per lane; one
  // 128 B load from half the lanes for the smallest tile).
  static constexpr int XW = XB / NW;
  static constexpr int XLB = XW >= 1024 ? 1024 : 256;  // bytes per token load
  static constexpr int XL = XW >= XLB ? XW / XLB : 1;
  static constexpr int LPS = WL + XL;            // loads per wave per stage
  static constexpr int PF = NW * NBT * MB * 256; // partial floats per workgroup
  static_assert(BK == 32 || BK == 64, "stage depth");
  static_assert(RP == 128 || RP == 256 || RP == 512, "region row");
  static_assert(WL >= 1 && RB % 1024 == 0 && (RB / 1024) % WL == 0, "a wave's loads stay in one region");
  static_assert(NST * SB <= 160 * 1024, "LDS");
};

// Swizzle masks (XOR on the 16-byte unit index of a row) that spread the
// fragment reads over distinct banks.  One transposing read takes 8 rows (two
// runs of 4 consecutive rows, 8 apart) per 32 lanes, which the mask sends to
// 8 distinct 32-byte bank groups; 256 and 512 B rows all start at bank 0.
// 128 B rows put two rows in one 256 B bank line, so there the mask takes
// four values per row parity.
template <int RP>
__device__ __forceinline__ int swz_w(int r) {
  if constexpr (RP == 128)
    return 2 * (((r >> 1) & 1) | (((r >> 3) & 1) << 1));
  else
    return 2 * ((r & 3) | (((r >> 3) & 1) << 2));
}
// Token rows are 128 or 64 B; one fragment read takes 16 consecutive rows per
// 16 lanes at one logical unit, which the mask sends to 16 distinct units.
template <int XP>
__device__ __forceinline__ int swz_x(int r) {
  if constexpr (XP == 128)
    return (r >> 1) & 7;
  else
    return (r >> 2) & 3;
}

struct DecodePlan {
  int64_t nblk;  // column blocks
  int64_t S;     // k-ranges (split-K factor)
  int64_t kc;    // k per range (multiple of BK)
  int mb;        // 16-row token blocks (1, 2 or 4)
  bool half;     // SwiGLU HALF layout (gate and up in different waves)
  int bk;        // k rows per stage (32 or 64)
  int64_t pf;    // partial floats per workgroup
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
  pl.mb = a.M <= 16 ? 1 : (a.M <= 32 ? 2 : 4);
  // One matrix: 128 columns (256 B of each weight row), 64-row stages.
  // SwiGLU streams two matrices: up to 32 tokens the same 256 B runs with
  // 32-row stages (the bytes per stage, and so in flight per CU, of the
  // single-matrix case); for 64 tokens, whose split-K partials are 4x larger,
  // the HALF layout over 64 columns with 64-row stages, which halves the
  // partials' traffic for 128 B runs.
  pl.half = dual && pl.mb == 4;
  pl.bk = (dual && !pl.half) ? 32 : 64;
  const int64_t width = pl.half ? 64 : 128;
  pl.nblk = (a.N + width - 1) / width;
  pl.pf = (int64_t)8 * (dual && !pl.half ? 2 : 1) * pl.mb * 256;
  const int64_t BK = pl.bk;
  const int64_t stages = (a.K + BK - 1) / BK;
  int64_t S = TARGET_WGS / pl.nblk;
  int64_t smax = stages / MIN_STAGES;
  if (smax < 1) smax = 1;
  if (S > smax) S = smax;
  if (S < 1) S = 1;
  if (split_override() > 0) S = split_override();
  const int64_t per = (stages + S - 1) / S;
  pl.kc = per * BK;
  pl.S = (a.K + pl.kc - 1) / pl.kc;
  return pl;
}

size_t ctr_bytes(int64_t nblk) { return ((size_t)nblk * 4 + CTR_BYTES - 1) / CTR_BYTES * CTR_BYTES; }

size_t plan_ws_bytes(const DecodePlan &pl) {
  if (pl.S <= 1) return 0;
  return ctr_bytes(pl.nblk) + (size_t)pl.nblk * pl.S * pl.pf * sizeof(float);
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
    if (p.bias) bv = (float)((const bf16 *)p.bias)[col];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t row = 16 * m + 4 * (lane >> 4) + v;
      if (row >= p.M) continue;
      if constexpr (EPI == EPI_SWIGLU)
        ((bf16 *)p.C)[row * p.ldc + col] = to_bf16(silu(acc[m][v]) * up[m][v]);
      else if constexpr (EPI == EPI_F32)
        ((float *)p.C)[row * p.ldc + col] = acc[m][v];
      else
        ((bf16 *)p.C)[row * p.ldc + col] = to_bf16(activate<ACT>(acc[m][v] + bv));
    }
}

template <int EPI, int ACT, int MB, bool HALF, int BK, int NW>
__global__ __launch_bounds__(NW * 64) void gemm_bf16_decode_kernel(const GemmArgs p, int64_t nblk,
                                                                   int64_t S, int64_t kc,
                                                                   unsigned *ctr, float *parts) {
  using G = Geo<EPI, HALF, MB, BK, NW>;
  constexpr bool DUAL = (EPI == EPI_SWIGLU);
  __shared__ __attribute__((aligned(1024))) char smem[NST * G::SB];
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t blk = blockIdx.x % nblk, s = blockIdx.x / nblk;
  const int64_t M = p.M, N = p.N;
  const int64_t kbeg = s * kc;
  const int64_t kend = (kbeg + kc < p.K) ? kbeg + kc : p.K;
  const int nstages = (int)((kend - kbeg + BK - 1) / BK);
  const int64_t n0 = blk * G::RC;  // first column of the block in every region

  // ---- per-lane load offsets, relative to a stage's k base -----------------
  // Weight load gi = WL w + j fills 1 KiB of region gi / LPR: RPL rows of RP
  // bytes; lane -> row (gi % LPR) RPL + lane / UPR, physical unit lane % UPR.
  constexpr int UPR = G::RP / 16;     // 16-byte units per region row
  constexpr int LPR = G::RB / 1024;   // loads per region
  const int wreg = (G::WL * wave) / LPR;
  const bf16 *Wm = (const bf16 *)(wreg ? p.B2 : p.B);
  const int64_t ldw = wreg ? p.ldb2 : p.ldb;
  uint32_t w_off[G::WL];
  int w_row[G::WL];
#pragma unroll
  for (int j = 0; j < G::WL; ++j) {
    const int li = (G::WL * wave + j) % LPR;
    const int r = li * G::RPL + lane / UPR;
    const int lu = (lane % UPR) ^ swz_w<G::RP>(r);
    const int64_t col = n0 + 8 * lu;
    w_row[j] = r;
    w_off[j] = col < N ? (uint32_t)((r * ldw + col) * 2) : OOB;
  }
  // Token rows: wave w fills bytes [XW w, XW (w+1)) of the token region, load
  // j the XLB bytes from XW w + XLB j; lane -> physical byte (XLB / 64) lane.
  uint32_t x_off[G::XL];
  int x_k[G::XL];
#pragma unroll
  for (int j = 0; j < G::XL; ++j) {
    const int pb = G::XW * wave + G::XLB * j + (G::XLB / 64) * lane;  // physical byte
    const int r = pb / G::XP, b = pb % G::XP;
    const int k = 8 * ((b >> 4) ^ swz_x<G::XP>(r)) + ((b & 15) >> 1);
    x_k[j] = k;
    x_off[j] = (r < M && r < 16 * MB) ? (uint32_t)((r * p.lda + k) * 2) : OOB;
  }
  const bf16 *X = (const bf16 *)p.A;

  // Loads of stage t into its buffer; past the last stage every lane gets an
  // out-of-range offset, so nothing is read and no branch is needed.
  auto issue_stage = [&](int t) {
    char *st = smem + (t % NST) * G::SB;
    const bool live = t < nstages;
    const int64_t k0 = kbeg + (int64_t)(live ? t : 0) * BK;
    const i32x4 rw = rsrc(Wm + k0 * ldw);
    const i32x4 rx = rsrc(X + k0);
#pragma unroll
    for (int j = 0; j < G::WL; ++j) {
      const uint32_t off = (live && k0 + w_row[j] < kend) ? w_off[j] : OOB;
      dma16(rw, st + (G::WL * wave + j) * 1024, off);
    }
#pragma unroll
    for (int j = 0; j < G::XL; ++j) {
      const uint32_t off = (live && k0 + x_k[j] < kend) ? x_off[j] : OOB;
      char *dst = st + G::WB + G::XW * wave + G::XLB * j;
      if constexpr (G::XLB == 1024)
        dma16(rx, dst, off);
      else if (G::XW >= 256 || lane < G::XW / 4)
        dma4(rx, dst, off);
    }
  };

  // ---- fragment addresses ------------------------------------------------------
  // Block f (region f, or w / (NW/2) in the HALF layout) at slice kk, half h: the
  // 16-lane group g reads rows 32 kk + 8 g + 4 h + (lane % 16) / 4 at columns
  // cb + 4 (lane % 4); the transposing read hands lane i column cb + i of
  // those 4 rows.
  int w_rd[G::NBT][G::KS][2];
#pragma unroll
  for (int f = 0; f < G::NBT; ++f)
#pragma unroll
    for (int kk = 0; kk < G::KS; ++kk)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int j = lane & 15;
        const int r = 32 * kk + 8 * (lane >> 4) + 4 * h + (j >> 2);
        const int c = 16 * (HALF ? wave % (NW / 2) : wave) + 4 * (j & 3);
        const int rg = HALF ? wave / (NW / 2) : f;
        w_rd[f][kk][h] =
            rg * G::RB + r * G::RP + (((c >> 3) ^ swz_w<G::RP>(r)) << 4) + ((c & 4) << 1);
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

  f32x4 acc[G::NBT][MB];
#pragma unroll
  for (int f = 0; f < G::NBT; ++f)
#pragma unroll
    for (int m = 0; m < MB; ++m) acc[f][m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // ---- the stream ----------------------------------------------------------------
#pragma unroll
  for (int t = 0; t < NST - 1; ++t) issue_stage(t);
  for (int t = 0; t < nstages; ++t) {
    // This wave's loads of stage t have landed (the next stage's may still be
    // in flight); after the barrier every wave's have, and every wave is done
    // reading stage t-1, whose buffer the next loads reuse.
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0((NST - 2) * G::LPS));
    wg_barrier();
    issue_stage(t + NST - 1);
    const char *st = smem + (t % NST) * G::SB;
#pragma unroll
    for (int kk = 0; kk < G::KS; ++kk) {
      bf16x8 xa[MB];
#pragma unroll
      for (int m = 0; m < MB; ++m) xa[m] = *(const bf16x8 *)(st + x_rd[m][kk]);
#pragma unroll
      for (int f = 0; f < G::NBT; ++f) {
        const s16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(st + w_rd[f][kk][0]));
        const s16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(st + w_rd[f][kk][1]));
        const s16x8 bv = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
#pragma unroll
        for (int m = 0; m < MB; ++m)
          acc[f][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[m], __builtin_bit_cast(bf16x8, bv),
                                                              acc[f][m], 0, 0, 0);
      }
    }
  }
  // The loads issued past the last stage read nothing but still write LDS:
  // none may be pending when the workgroup ends.
  __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));

  // Output column of this lane; in the HALF layout the gate waves write.
  const int64_t col = n0 + 16 * (HALF ? wave % (NW / 2) : wave) + (lane & 15);
  const bool up_wave = HALF && wave >= NW / 2;
  if (S == 1) {
    if constexpr (HALF) {
      // Hand the up sums to the gate waves through LDS.
      wg_barrier();
      f32x4 *xch = (f32x4 *)smem;
      if (up_wave) {
#pragma unroll
        for (int m = 0; m < MB; ++m) xch[((wave - NW / 2) * MB + m) * 64 + lane] = acc[0][m];
      }
      __syncthreads();
      if (up_wave) return;
      f32x4 up[MB];
#pragma unroll
      for (int m = 0; m < MB; ++m) up[m] = xch[(wave * MB + m) * 64 + lane];
      store_out<EPI, ACT, MB>(p, col, lane, acc[0], up);
    } else {
      store_out<EPI, ACT, MB>(p, col, lane, acc[0], acc[DUAL ? 1 : 0]);
    }
    return;
  }

  // ---- split-K: publish the partial; the last arriver reduces --------------------
  // Partials are written and read as agent-scope atomics, which the hardware
  // keeps coherent across the XCDs' L2 caches without a cache write-back or
  // invalidate; a wave's stores have completed once vmcnt reaches zero, before
  // the barrier that precedes the counter update.
  // Token rows past M (padding) are neither written nor read.
  constexpr int NV = G::NBT * MB * 4;  // floats per lane
  float *base = parts + blk * S * G::PF + (int64_t)wave * (NV * 64) + lane;
  {
    float *mine = base + s * G::PF;
#pragma unroll
    for (int f = 0; f < G::NBT; ++f)
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (16 * m + 4 * (lane >> 4) + v < M)
            __hip_atomic_store(mine + ((f * MB + m) * 4 + v) * 64, acc[f][m][v], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(wait_vm(0));
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(ctr + blk, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (unsigned)(S - 1);
  }
  __syncthreads();
  if (!s_last || up_wave) return;

  // Partials are read RCH ranges at a time, all loads of a chunk issued before
  // any is added (ranges past S read the last one again and add nothing), and
  // summed in k-range order.
  // In the HALF layout a gate wave also reads the slot of its up partner.
  constexpr int NF = HALF ? 2 : G::NBT;  // blocks summed per lane
  constexpr int NVR = NF * MB * 4;       // floats read per lane per range
  constexpr int RCH = NVR > 32 ? 2 : 4;
  f32x4 sum[NF][MB];
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int m = 0; m < MB; ++m) sum[f][m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int64_t s2 = 0; s2 < S; s2 += RCH) {
    float val[RCH][NVR];
#pragma unroll
    for (int c = 0; c < RCH; ++c) {
      const int64_t sc = (s2 + c < S) ? s2 + c : S - 1;
      const float *ps = base + sc * G::PF;
#pragma unroll
      for (int e = 0; e < NVR; ++e) {
        const int f = e / (MB * 4), m = (e / 4) % MB, v = e % 4;
        // HALF: block 1 is the partner wave's slot, NW/2 waves further on.
        const int off = HALF ? f * (NW / 2) * NV * 64 + (e % (MB * 4)) * 64 : e * 64;
        val[c][e] = (16 * m + 4 * (lane >> 4) + v < M)
                        ? __hip_atomic_load(ps + off, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                        : 0.0f;
      }
    }
#pragma unroll
    for (int c = 0; c < RCH; ++c) {
      if (s2 + c >= S) break;
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
          for (int v = 0; v < 4; ++v) sum[f][m][v] += val[c][(f * MB + m) * 4 + v];
    }
  }
  if (tid == 0) __hip_atomic_store(ctr + blk, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  store_out<EPI, ACT, MB>(p, col, lane, sum[0], sum[DUAL ? 1 : 0]);
}

template <int EPI, int ACT, int MB, bool HALF, int BK>
hipError_t launch_plan(const GemmArgs &a, const DecodePlan &pl, void *ws, hipStream_t st) {
  unsigned *ctr = nullptr;
  float *parts = nullptr;
  if (pl.S > 1) {
    ctr = (unsigned *)ws;
    parts = (float *)((char *)ws + ctr_bytes(pl.nblk));
  }
  hipLaunchKernelGGL((gemm_bf16_decode_kernel<EPI, ACT, MB, HALF, BK, NWAVE>),
                     dim3((unsigned)(pl.nblk * pl.S)), dim3(NWAVE * 64), 0, st, a, pl.nblk, pl.S,
                     pl.kc, ctr, parts);
  return hipGetLastError();
}

template <int EPI, int ACT>
hipError_t launch_mb(const GemmArgs &a, const DecodePlan &pl, void *ws, hipStream_t st) {
  // The configurations make_plan chooses.
  constexpr bool DUAL = EPI == EPI_SWIGLU;
  switch (pl.mb) {
    case 1:
      return launch_plan<EPI, ACT, 1, false, DUAL ? 32 : 64>(a, pl, ws, st);
    case 2:
      return launch_plan<EPI, ACT, 2, false, DUAL ? 32 : 64>(a, pl, ws, st);
    default:
      return launch_plan<EPI, ACT, 4, DUAL, 64>(a, pl, ws, st);
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
  // 64 weight rows and 64 token rows must stay below 2^31 bytes.
  return a.M >= 1 && a.M <= 64 && a.lda < (int64_t(1) << 23) && a.ldb < (int64_t(1) << 23) &&
         (a.epi != EPI_SWIGLU || a.ldb2 < (int64_t(1) << 23));
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
