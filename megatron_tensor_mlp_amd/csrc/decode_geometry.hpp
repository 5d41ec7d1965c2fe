// Addressing of the few-token GEMM (gemm_decode.hip): which column block and
// k-range a workgroup takes, where each lane's buffer-to-LDS loads read, the
// split-K partial slots, and the output coordinates.  Host and device share
// these functions: the kernel computes its addresses with them, and a
// host-side bounds model runs the same code over every workgroup, wave and
// lane of a launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace tpmlp {
namespace decode {

constexpr int NWAVE = 8;
constexpr int RC = 16 * NWAVE;  // columns per workgroup
constexpr int RP = RC * 2;      // bytes per weight row in LDS
constexpr uint32_t OOB_OFF = 0x80000000u;  // an offset past every buffer range

// Swizzle mask (XOR on the 16-byte unit index of a row) that spreads the
// fragment reads over distinct banks: one transposing read takes 8 rows (two
// runs of 4 consecutive rows, 8 apart) per 32 lanes, and 256 B rows all start
// at bank 0, so the mask sends those rows to 8 distinct 32-byte bank groups.
__host__ __device__ __forceinline__ int swz_w(int r) {
  return 2 * ((r & 3) | (((r >> 3) & 1) << 2));
}
// Token rows are 128 or 64 B; one fragment read takes 16 consecutive rows per
// 16 lanes at one logical unit, which the mask sends to 16 distinct units.
template <int XP>
__host__ __device__ __forceinline__ int swz_x(int r) {
  if constexpr (XP == 128)
    return (r >> 1) & 7;
  else
    return (r >> 2) & 3;
}

// Geometry of one configuration: a stage holds BK k rows of 128 columns and
// the matching token rows (16 MB of them, MB token blocks).
template <int MB, int BK, int NST>
struct Geo {
  static constexpr int KS = BK / 32;             // 32-k MFMA slices per stage
  static constexpr int WB = BK * RP;             // weight bytes per stage
  static constexpr int XP = BK * 2;              // bytes per token row
  static constexpr int XB = 16 * MB * XP;        // token bytes per stage
  static constexpr int SB = WB + XB;             // stage bytes
  static constexpr int WL = WB / 1024 / NWAVE;   // 1 KiB weight loads per wave per stage
  // Token rows: XB / 8 bytes per wave, in 1 KiB loads (16 B per lane) when
  // there are at least that many, else in 256 B loads (4 B per lane; one
  // 128 B load from half the lanes for the smallest tile).
  static constexpr int XW = XB / NWAVE;
  static constexpr int XLB = XW >= 1024 ? 1024 : 256;
  static constexpr int XL = XW >= XLB ? XW / XLB : 1;
  static constexpr int LPS = WL + XL;            // loads per wave per stage
  static constexpr int PF = NWAVE * MB * 256;    // partial floats per workgroup (one slot)
  static_assert(BK == 32 || BK == 64, "stage depth");
  static_assert(WL >= 1, "loads");
  static_assert(NST >= 3 && NST * SB <= 160 * 1024, "LDS");

  // Weight load gi = WL wave + j fills 1 KiB = 4 rows of 256 B; lane -> row
  // 4 gi + lane / 16, physical unit lane % 16.  row: the k row (relative to
  // the stage's base); off: byte offset from that base, OOB_OFF for columns
  // past N.
  __host__ __device__ static __forceinline__ void w_load(const GemmArgs &p, int64_t ldw,
                                                         int64_t n0, int wave, int lane, int j,
                                                         uint32_t &off, int &row) {
    const int r = 4 * (WL * wave + j) + lane / 16;
    const int lu = (lane % 16) ^ swz_w(r);
    const int64_t col = n0 + 8 * lu;
    row = r;
    off = col < p.N ? (uint32_t)((r * ldw + src_col(p, col)) * 2) : OOB_OFF;
  }
  // Token rows: wave w fills bytes [XW w, XW (w+1)) of the token region, load
  // j the XLB bytes from XW w + XLB j; lane -> physical byte (XLB / 64) lane.
  // k: the first k (relative to the stage) of the lane's bytes; off: byte
  // offset from the stage's base, OOB_OFF for rows past M.
  __host__ __device__ static __forceinline__ void x_load(const GemmArgs &p, int wave, int lane,
                                                         int j, uint32_t &off, int &k) {
    const int pb = XW * wave + XLB * j + (XLB / 64) * lane;  // physical byte
    const int r = pb / XP, b = pb % XP;
    k = 8 * ((b >> 4) ^ swz_x<XP>(r)) + ((b & 15) >> 1);
    off = (r < p.M && r < 16 * MB) ? (uint32_t)((r * p.lda + k) * 2) : OOB_OFF;
  }
  // Whether the lane takes part in token load j (the smallest tile loads
  // 128 B from half the lanes).
  __host__ __device__ static __forceinline__ bool x_lane(int lane) {
    return XLB == 1024 || XW >= 256 || lane < XW / 4;
  }
  // Bytes one lane's token load moves.
  static constexpr int X_BYTES = XLB == 1024 ? 16 : 4;
  // LDS byte offsets within a stage of weight load j and token load j.
  __host__ __device__ static __forceinline__ int w_lds(int wave, int j) {
    return (WL * wave + j) * 1024;
  }
  __host__ __device__ static __forceinline__ int x_lds(int wave, int j) {
    return WB + XW * wave + XLB * j;
  }
  // The offset a load of stage t uses: its lane's offset while the stage
  // exists (live) and the lane's first k lies below the range's end, else
  // OOB_OFF.
  __host__ __device__ static __forceinline__ uint32_t stage_off(bool live, int64_t k0, int k,
                                                                int64_t kend, uint32_t off) {
    return (live && k0 + k < kend) ? off : OOB_OFF;
  }

  // Split-K partials: a slot holds [wave][m][lane] 16-byte groups (lane
  // accumulator block m: rows 16 m + 4 (lane / 16) + 0..3 of column lane %
  // 16); groups with no token row below M are neither written nor read.
  __host__ __device__ static __forceinline__ uint32_t group_off(int64_t M, int wave, int lane,
                                                                int m) {
    return (16 * m + 4 * (lane >> 4) < M) ? (uint32_t)(((wave * MB + m) * 64 + lane) * 16)
                                          : OOB_OFF;
  }
  // Byte offset of slot (q, s) from the block's first slot: the S gate (or
  // only) partials in k-range order, then the S up partials.
  __host__ __device__ static __forceinline__ uint32_t slot_off(int q, int64_t S, int64_t s) {
    return (uint32_t)((q * S + s) * (PF * 4));
  }
  // Floats of a column block's slots (nparts = NMAT * S of them).
  __host__ __device__ static __forceinline__ int64_t block_floats(int64_t nparts) {
    return nparts * PF;
  }
};

// Workgroup b's column block and k-range.  Grid order: for each k-range, the
// gate column blocks, then the up ones.
__host__ __device__ __forceinline__ void wg_coords(int64_t bid, int nmat, int64_t nblk,
                                                   int64_t &blk, int64_t &s, bool &up) {
  const int64_t wide = bid % (nmat * nblk);
  s = bid / (nmat * nblk);
  up = nmat == 2 && wide >= nblk;
  blk = up ? wide - nblk : wide;
}
// The k-range [kbeg, kend) of range s.
__host__ __device__ __forceinline__ void k_range(int64_t s, int64_t kc, int64_t K, int64_t &kbeg,
                                                 int64_t &kend) {
  kbeg = s * kc;
  kend = (kbeg + kc < K) ? kbeg + kc : K;
}
// Output coordinates: wave w's 16-column block, lane column (lane & 15); rows
// 16 m + 4 (lane / 16) + v of accumulator block m.
__host__ __device__ __forceinline__ int64_t out_col(int64_t n0, int wave, int lane) {
  return n0 + 16 * wave + (lane & 15);
}
__host__ __device__ __forceinline__ int64_t out_row(int m, int lane, int v) {
  return 16 * m + 4 * (lane >> 4) + v;
}

}  // namespace decode
}  // namespace tpmlp
