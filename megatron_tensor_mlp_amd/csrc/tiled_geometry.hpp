// Addressing of the tiled bf16 GEMM (gemm_tiled.hip): which tile a workgroup
// takes, where each lane's buffer-to-LDS loads read, and where the epilogue's
// accumulator elements land.  Host and device share these functions: the kernel
// computes its addresses with them, and a host-side bounds model runs the same
// code over every workgroup, wave and lane of a launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace tpmlp {
namespace tiled {

constexpr int BN = 256;               // tile columns (SwiGLU: 128 gate + 128 up)
constexpr int GROUP_M = 4;            // row-tiles walked together for L2 reuse
constexpr uint32_t OOB_OFF = 0x80000000u;  // an offset past every buffer range: reads as zero

// XOR masks on the 16-byte unit index of an LDS row.
//  A rows (2*BK bytes = BK/8 units): fragment reads touch 8 or 16 consecutive
//  rows at one logical unit; the mask spreads them over distinct banks.
template <int BK>
__host__ __device__ __forceinline__ int swz_a(int r) {
  if constexpr (BK == 64)
    return ((r >> 1) ^ (r << 2)) & 7;
  else
    return ((r >> 1) ^ (r >> 2)) & 3;
}
//  B rows (512 or 256 B): a transposing read touches 4 consecutive k rows x
//  32 or 64 bytes; rows k..k+3 get masks 0, 4, 10, 14 (distinct 64-byte
//  segments and distinct 32-byte pairs within them).
__host__ __device__ __forceinline__ int swz_b(int k) { return ((k & 3) << 2) ^ (k & 2); }

// Workgroup b runs on XCD b % 8.  Give every XCD a contiguous run of the tile
// order (a bijection for any total), then walk GROUP_M row-tiles at a time so
// the tiles resident on one XCD share A and B panels in its L2.
__host__ __device__ __forceinline__ void tile_coords(int bid, int tilesM, int tilesN, int total,
                                                     int &g, int &tm, int &tn) {
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

// Split-K: workgroup b of a launch of `total` tiles times S k-ranges takes
// tile b % total (in the order above; with total a multiple of 8 the tile's
// XCD is still b % 8) and k-range b / total.  The ranges are kc long, kc =
// ceil(K / S) rounded up to a whole k-step, the last one ragged; a launch
// takes S = ceil(K / kc) ranges, for which the same formula gives back kc.
__host__ __device__ __forceinline__ void split_coords(int bid, int total, int &tile, int &sidx) {
  tile = bid % total;
  sidx = bid / total;
}
__host__ __device__ __forceinline__ int64_t split_kc(int64_t K, int S, int BK) {
  const int64_t per = (K + S - 1) / S;
  return (per + BK - 1) / BK * BK;
}
__host__ __device__ __forceinline__ void split_range(int64_t K, int64_t kc, int sidx,
                                                     int64_t &kbeg, int64_t &kend) {
  kbeg = (int64_t)sidx * kc;
  kend = kbeg + kc < K ? kbeg + kc : K;
}

// Geometry of one kernel configuration: BK k per step, NWAVE waves, BM tile
// rows, DUAL (SwiGLU: gate and up regions), LAY (operand layout).
template <int BK, int NWAVE, int BM, bool DUAL, int LAY>
struct Geom {
  static constexpr bool TA = (LAY == LAY_TN);  // A held as A^T [K,M]: m contiguous
  static constexpr bool TB = (LAY == LAY_NT);  // B held as B^T [N,K]: k contiguous
  static constexpr int NOUT = DUAL ? BN / 2 : BN;       // output columns per tile
  static constexpr int WMW = BM / 128;                  // waves along M (128 rows each)
  static constexpr int WNW = NWAVE / WMW;               // waves along N
  static constexpr int WN = BN / WNW;                   // accumulator columns per wave
  static constexpr int NB = WN / 32;                    // 32-column B fragments per wave
  static constexpr int A_BYTES = BM * BK * 2;           // [BM rows][BK k]
  static constexpr int B_BYTES = BK * BN * 2;           // [BK k][256 cols] or 2 x [BK][128]
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int AUNITS = BK / 8;                 // 16-byte units per k-contiguous row
  static constexpr int AROWS_PER_LOAD = 64 / AUNITS;    // k-contiguous rows one 1 KiB load fills
  static constexpr int APITCH = TA ? 2 * BM : 2 * BK;   // bytes per A row in LDS (k rows when TA)
  static constexpr int ATUNITS = BM / 8;                // 16-byte units per k row of A^T
  static constexpr int AKROWS_PER_LOAD = 1024 / APITCH; // k rows of A^T one load fills
  static constexpr int A_LOADS = A_BYTES / 1024 / NWAVE;  // per wave
  static constexpr int BREG = DUAL ? BN / 2 : BN;       // columns per B region
  static constexpr int BPITCH = BREG * 2;               // bytes per B row
  static constexpr int BUNITS = BREG / 8;               // 16-byte units per B row
  static constexpr int BROWS_PER_LOAD = 1024 / BPITCH;  // B rows one wave-wide load fills
  static constexpr int B_LOADS = B_BYTES / 1024 / NWAVE;  // per wave
  static constexpr int B_LOADS_PER_REGION = (B_BYTES / 1024) / (DUAL ? 2 : 1);
  static constexpr int LPS = A_LOADS + B_LOADS;         // loads per wave per stage

  // Base of the tile's A panel (element pointer; T is the element type).
  template <typename T>
  __host__ __device__ static __forceinline__ const T *a_tile(const GemmArgs &p, int g,
                                                             int64_t m0) {
    return (const T *)p.A + g * p.sA + (TA ? m0 : m0 * p.lda);
  }
  // Group bases of the gate (or only) and up matrices.  B offsets are taken
  // from the matrix base: a column map may send a tile's columns to separate
  // column blocks of B.
  template <typename T>
  __host__ __device__ static __forceinline__ const T *b_group(const GemmArgs &p, int g) {
    return (const T *)p.B + g * p.sB;
  }
  template <typename T>
  __host__ __device__ static __forceinline__ const T *b2_group(const GemmArgs &p, int g) {
    return DUAL ? (const T *)p.B2 + g * p.sB2 : nullptr;
  }
  // Waves in the second half of the B loads fill the up region.
  __host__ __device__ static __forceinline__ bool b_up(int wave) {
    return DUAL && (B_LOADS * wave >= B_LOADS_PER_REGION);
  }

  // A load j of `wave`: load j fills rows (A_LOADS wave + j) * AROWS_PER_LOAD +
  // lane / AUNITS, physical unit lane % AUNITS (logical unit = physical ^
  // swizzle).  off: byte offset from the k-step's base, OOB_OFF for rows past
  // M; kof: the first k (relative to the step) that the lane's 16 bytes hold.
  __host__ __device__ static __forceinline__ void a_load(const GemmArgs &p, int64_t m0, int wave,
                                                         int lane, int j, uint32_t &off,
                                                         int &kof) {
    if constexpr (!TA) {
      const int r = (A_LOADS * wave + j) * AROWS_PER_LOAD + lane / AUNITS;
      const int lu = (lane % AUNITS) ^ swz_a<BK>(r);
      kof = 8 * lu;
      off = (m0 + r < p.M) ? (uint32_t)((r * p.lda + 8 * lu) * 2) : OOB_OFF;
    } else {
      // A^T: load j fills k rows (A_LOADS w + j) * AKROWS_PER_LOAD + lane / ATUNITS
      // of BM m each; lane -> physical unit lane % ATUNITS.
      const int k = (A_LOADS * wave + j) * AKROWS_PER_LOAD + lane / ATUNITS;
      const int lu = (lane % ATUNITS) ^ swz_b(k);
      kof = k;
      off = (m0 + 8 * lu < p.M) ? (uint32_t)((k * p.lda + 8 * lu) * 2) : OOB_OFF;
    }
  }

  // B load j of `wave` is load gi = B_LOADS wave + j of the tile, filling
  // 1 KiB of a B region = BROWS_PER_LOAD rows; lane -> row lane / BUNITS, unit
  // lane % BUNITS.  With SwiGLU the first half of the loads fill the gate
  // region and the second half the up region.  off as for A (OOB_OFF for
  // columns past N); k: the k (relative to the step) of the lane's first
  // element.
  __host__ __device__ static __forceinline__ void b_load(const GemmArgs &p, int64_t n0, int wave,
                                                         int lane, int j, uint32_t &off,
                                                         int &k) {
    const int gi = B_LOADS * wave + j;
    const int li = gi % B_LOADS_PER_REGION;
    const int64_t ld = b_up(wave) ? p.ldb2 : p.ldb;
    if constexpr (!TB) {
      const int kr = li * BROWS_PER_LOAD + lane / BUNITS;
      const int lu = (lane % BUNITS) ^ swz_b(kr);
      const int64_t col = n0 + 8 * lu;  // output column of this 16-byte unit
      k = kr;
      off = (col < p.N) ? (uint32_t)((kr * ld + src_col(p, col)) * 2) : OOB_OFF;
    } else {
      // B^T: load j fills n rows li * AROWS_PER_LOAD + lane / AUNITS of the
      // region, BK k each, like the rows of A.
      const int r = li * AROWS_PER_LOAD + lane / AUNITS;
      const int lu = (lane % AUNITS) ^ swz_a<BK>(r);
      const int64_t col = n0 + r;  // output column of this row
      k = 8 * lu;
      off = (col < p.N) ? (uint32_t)((src_col(p, col) * ld + 8 * lu) * 2) : OOB_OFF;
    }
  }

  // The offset a load of k-step k0 uses: its lane's offset while the step
  // exists (live) and the lane's first k lies below K, else OOB_OFF (zeros,
  // no memory touched).
  __host__ __device__ static __forceinline__ uint32_t step_off(bool live, int64_t k0, int kof,
                                                               int64_t K, uint32_t off) {
    return (live && k0 + kof < K) ? off : OOB_OFF;
  }
  // LDS byte offsets within a stage that A load q and B load j of `wave` fill
  // (1 KiB each; the B regions follow A and each other).
  __host__ __device__ static __forceinline__ int a_lds(int wave, int q) {
    return (A_LOADS * wave + q) * 1024;
  }
  __host__ __device__ static __forceinline__ int b_lds(int wave, int j) {
    return A_BYTES + (B_LOADS * wave + j) * 1024;
  }

  // Bases of k-step k0 (the buffer descriptors' base addresses).
  template <typename T>
  __host__ __device__ static __forceinline__ const T *a_step(const GemmArgs &p, const T *A,
                                                             int64_t k0) {
    return TA ? A + k0 * p.lda : A + k0;
  }
  template <typename T>
  __host__ __device__ static __forceinline__ const T *b_step(const GemmArgs &p, const T *B,
                                                             const T *B2, bool up, int64_t k0) {
    if constexpr (TB)  // k past ksplit comes from the second matrix (same ld)
      return p.ksplit > 0 && k0 >= p.ksplit ? (const T *)p.B2 + (k0 - p.ksplit)
                                             : (up ? B2 : B) + k0;
    else
      return up ? B2 + k0 * p.ldb2 : B + k0 * p.ldb;
  }

  // Epilogue: the 32x32 accumulator layout gives lane the column (lane & 31)
  // and rows 8 (v / 4) + 4 (lane / 32) + (v % 4), v = 0..15, of fragment
  // (i, f) of the wave at (wm, wn).  Output column of fragment f (SwiGLU: of
  // its gate half).
  __host__ __device__ static __forceinline__ int64_t out_col(int64_t n0, int wn, int f, int lane) {
    return n0 + (DUAL ? WN / 2 : WN) * wn + 32 * f + (lane & 31);
  }
  // Split-K partial slots: one per (tile, k-range), tile-major, each holding
  // every wave's accumulators as 16-byte groups [wave][i][f][quarter q][lane]
  // (q: accumulator elements 4q..4q+3), so one store or load instruction of a
  // wave covers 1 KiB.  part_off: a group's byte offset within its slot.
  static constexpr int64_t SLOT_BYTES = (int64_t)NWAVE * 4 * NB * 4 * 64 * 16;
  __host__ __device__ static __forceinline__ uint32_t part_off(int wave, int lane, int i, int f,
                                                               int q) {
    return (uint32_t)(((((wave * 4 + i) * NB + f) * 4 + q) * 64 + lane) * 16);
  }

  __host__ __device__ static __forceinline__ int64_t row_base(int64_t m0, int wm, int lane) {
    return m0 + 128 * wm + 4 * (lane >> 5);
  }
  __host__ __device__ static __forceinline__ int64_t out_row(int64_t rbase, int i, int v) {
    return rbase + 32 * i + 8 * (v >> 2) + (v & 3);
  }
};

}  // namespace tiled
}  // namespace tpmlp
