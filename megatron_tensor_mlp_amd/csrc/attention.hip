// Attention core of one head shard for gfx950: per query head,
// O = softmax(Q K^T / sqrt(dh)) V over the keys each query sees (causal or
// not), with grouped key/value heads ("Transformer math: tensor parallel",
// section "Attention: parallel across heads": heads never mix, so a GPU runs
// full attention for its own heads with no communication).
//
// Work units.  A workgroup owns HPW query heads that read the same key/value
// head (HPW = 4, 2 or 1, the largest that divides the query heads per
// key/value head), so that every key and value tile it brings into LDS serves
// HPW heads: the tiles of one key/value head are what the whole launch reads
// over and over (from L2), and sharing them divides that traffic by HPW.  The
// queries of a sequence form N blocks of 64/HPW; each of the 4 waves of a
// group owns 16 queries of one of the HPW heads.  The workgroup owns two
// blocks, j and N-1-j, so that under the causal mask every workgroup has the
// same number of key tiles (blocks near the start see few keys, those near
// the end many).  The pair's key tiles form one list, block j's tiles then
// block N-1-j's.  Group 0 (waves 0-3) walks the first half of the list and
// group 1 (waves 4-7) the second half from its end, so both groups do the
// same number of tiles with two waves on every SIMD; the block whose tiles the
// halves share is finished by merging the two partial softmax states
// (maximum, sum, unnormalised output) through LDS.  Key and value tiles of 64
// keys go from HBM to LDS by buffer loads that write LDS directly,
// double-buffered per group; the key stream runs one tile ahead of the value
// stream so that the MFMAs of the next tile's scores overlap the current
// tile's exponentials.
//
// The scores are computed transposed, S^T = K Q^T, with
// v_mfma_f32_16x16x32_bf16: K is the A operand (16-byte LDS reads of 8
// consecutive head dimensions), Q^T the B operand (each lane's 8 head
// dimensions of its query, held in registers).  In the accumulator layout
// every lane then holds 4 keys of ONE query, so the softmax state is
// lane-local, up to a reduction over the 4 lanes that share a query.  The
// output is accumulated transposed too, O^T += V^T P^T: P^T is the B operand
// straight from the score registers (rounded to bf16), and V^T the A operand,
// read from the [key][dh] tile with the transposing LDS read; the MFMA's
// k-index runs over the keys in the order the score registers hold them
// (keys 4g..4g+3 and 16+4g..16+4g+3 for lane group g), which both operands
// follow, so the sum is unchanged.
//
// Softmax arithmetic.  Base 2: the exponent of a score s is
// s * log2(e)/sqrt(dh) - m, one fused multiply-add, then v_exp_f32 (results
// below 2^-126 flush to zero, which no softmax weight of a bf16 product can
// feel next to the maximum's weight of at least 1).  The reference m moves
// only when a tile's maximum exceeds it by more than 8 (a factor 256), so the
// weights stay below 256 and the output is rescaled a few times per query
// instead of once per tile; the result is the same quotient, since every
// weight and the running sum share the one reference.  Only tiles that cross
// the causal diagonal or the end of the sequence compare key indices.
#include "device_common.hpp"
#include "kernels.h"
#include "lds_dma.hpp"

namespace tpmlp {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

constexpr int KT = 64;          // keys per tile
constexpr float LAZY = 8.0f;    // the reference maximum may lag the true one by this (log2 units)

// XOR swizzles on the 16-byte unit index of a tile row (DH*2 bytes).
//  K rows: a 16-byte fragment read takes 16 consecutive rows at one logical
//  unit per 16 lanes; the mask sends them to 16 distinct units.
template <int DH>
__device__ __forceinline__ int swz_k(int r) {
  return r & (DH / 8 - 1);
}
//  V rows: a transposing read takes 4 consecutive rows x 32 bytes per 16
//  lanes; the mask (even, so a 32-byte pair of units stays a pair) sends the
//  4 rows to distinct 32-byte segments, and with 16-unit rows the next 4 rows
//  to the other half of the row.
template <int DH>
__device__ __forceinline__ int swz_v(int r) {
  return (2 * (r & 3)) ^ (DH == 128 ? ((r >> 2) & 1) * 8 : 0);
}

// Reductions over the 4 rows of 16 lanes (the 4 lanes that hold keys of one
// query), the result in every lane: v_permlane16_swap exchanges rows 1 and 3
// of one copy with rows 0 and 2 of the other, v_permlane32_swap the two
// 32-lane halves; both are plain VALU instructions, no LDS round trip.
__device__ __forceinline__ float rows_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

constexpr int NGRP = 2;  // groups of 4 waves per workgroup

template <int DH, bool CAUSAL, int HPW>
__global__ __launch_bounds__(NGRP * 256, 1) void attention_kernel(AttnArgs p) {
  constexpr int QB = 64 / HPW;                  // queries per block and head
  constexpr int UNITS = DH / 8;                 // 16-byte units per tile row
  constexpr int TILE = KT * DH * 2;             // bytes of one K (or V) tile
  constexpr int LOADS = TILE / 1024 / 4;        // 1 KiB loads per wave per tile
  constexpr int ROWS_PER_LOAD = 1024 / (DH * 2);
  constexpr int DS = DH / 32;                   // 32-dh MFMA steps of the scores
  constexpr int DB = DH / 16;                   // 16-dh output blocks
  __shared__ __attribute__((aligned(1024))) char smem[NGRP][2][2][TILE];  // [group][buffer][K|V]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, gw = wave & 3;     // group, wave within the group
  const int hs = gw % HPW, qs = gw / HPW;       // the wave's head in the workgroup's set, and
                                                // its 16 queries within the block
  const int g4 = lane >> 4, l16 = lane & 15;
  const int S = (int)p.S;
  const int nblk = (S + QB - 1) / QB;
  const int npair = (nblk + 1) / 2;
  const int pair = (int)(blockIdx.x % npair);
  const int64_t hset = (blockIdx.x / npair) % (p.Hq / HPW);
  const int64_t h = hset * HPW + hs;            // this wave's query head
  const int64_t seq = blockIdx.x / ((int64_t)npair * (p.Hq / HPW));
  const int64_t c = hset * HPW / (p.Hq / p.Hkv);  // the key/value head all HPW heads read
  const bf16 *Qs = (const bf16 *)p.Q + seq * p.S * p.ldq + h * DH;
  const bf16 *Ks = (const bf16 *)p.K + seq * p.S * p.ldk + c * DH;
  const bf16 *Vs = (const bf16 *)p.V + seq * p.S * p.ldv + c * DH;
  bf16 *Os = (bf16 *)p.O + seq * p.S * p.ldo + h * DH;
  const float qk_scale = p.scale_log2;

  // The pair's tile list: items [0, na) are block a's tiles, [na, na+nb) block b's.
  auto ntiles_of = [&](int blk) {
    const int kend = CAUSAL ? min(blk * QB + QB, S) : S;
    return (kend + KT - 1) / KT;
  };
  const int blk_a = pair, blk_b = nblk - 1 - pair;
  const int na = ntiles_of(blk_a), nb = blk_b != blk_a ? ntiles_of(blk_b) : 0;
  const int total = na + nb;
  const int half = (total + 1) / 2;
  const bool split = half != na;                // a block's tiles are shared by the groups
  const int my_n = grp == 0 ? half : total - half;
  auto item_of = [&](int it) { return grp == 0 ? it : total - 1 - it; };

  // Per-lane DMA offsets inside a tile: load j of wave gw fills rows
  // (LOADS gw + j) * ROWS_PER_LOAD + lane / UNITS; physical unit lane % UNITS.
  int ld_row[LOADS], ld_ku[LOADS], ld_vu[LOADS];
#pragma unroll
  for (int j = 0; j < LOADS; ++j) {
    const int r = (LOADS * gw + j) * ROWS_PER_LOAD + lane / UNITS;
    ld_row[j] = r;
    ld_ku[j] = (lane % UNITS) ^ swz_k<DH>(r);
    ld_vu[j] = (lane % UNITS) ^ swz_v<DH>(r);
  }
  auto tile_k0 = [&](int it) {
    const int item = item_of(it);
    return (item < na ? item : item - na) * KT;
  };
  auto tile_blk = [&](int it) { return item_of(it) < na ? blk_a : blk_b; };
  // The key (which = 0) or value (which = 1) tile of the group's item `it`
  // into that operand's buffer `buf`.
  auto issue = [&](int it, int buf, int which) {
    const int k0 = tile_k0(it);
    const int64_t ld = which == 0 ? p.ldk : p.ldv;
    const i32x4 rs = rsrc((which == 0 ? Ks : Vs) + (int64_t)k0 * ld);
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const bool live = k0 + ld_row[j] < S;
      const int u = which == 0 ? ld_ku[j] : ld_vu[j];
      dma16(rs, smem[grp][buf][which] + (LOADS * gw + j) * 1024,
            live ? (uint32_t)((ld_row[j] * ld + 8 * u) * 2) : OOB);
    }
  };
  // Q^T fragments: 8 consecutive dh of the lane's query per 32-dh step.
  auto load_q = [&](bf16x8(&q)[DS], int blk) {
    const int qrow = blk * QB + 16 * qs + l16;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      if (qrow < S)
        q[s] = *(const bf16x8 *)(Qs + (int64_t)qrow * p.ldq + 32 * s + 8 * g4);
      else
        q[s] = bf16x8{};
    }
  };

  bf16x8 qf[DS], qf2[DS];  // Q^T of the block being scored; of the group's second block
  int qblk = -1;
  // Softmax state of block `cur` (this lane's query).
  f32x4 o[DB];
  float m_ref = -INFINITY, l_run = 0.0f;
  int cur = -1;

  // O = O^T / l: the lane holds dh rows 16 b + 4 g4 + v of its query.
  auto finish_block = [&](int blk) {
    const float l_tot = rows_sum(l_run);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const int qrow = blk * QB + 16 * qs + l16;
    if (qrow < S) {
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        const bf16x4 w = {to_bf16(o[b][0] * inv), to_bf16(o[b][1] * inv), to_bf16(o[b][2] * inv),
                          to_bf16(o[b][3] * inv)};
        *(bf16x4 *)(Os + (int64_t)qrow * p.ldo + 16 * b + 4 * g4) = w;
      }
    }
  };

  // Scores S^T [64 keys x 16 queries] of the key tile at kt, as 4 blocks of 16 keys.
  auto scores = [&](const char *kt, f32x4(&sc)[4]) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      sc[kb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      const int r = 16 * kb + l16;  // key row of this lane's A fragment
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        const int u = 4 * s + g4;
        const bf16x8 ka = *(const bf16x8 *)(kt + r * (DH * 2) + ((u ^ swz_k<DH>(r)) << 4));
        sc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[s], sc[kb], 0, 0, 0);
      }
    }
  };

  // Online softmax (base 2) of one tile's scores, then O^T += V^T P^T.
  auto softmax_pv = [&](f32x4(&sc)[4], const char *vt, int blk, int k0) {
    const int qw0 = blk * QB + 16 * qs;  // the wave's first query
    if ((CAUSAL && k0 + KT - 1 > qw0) || k0 + KT > S) {  // the diagonal or the sequence end
      const int qrow = qw0 + l16;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int key = k0 + 16 * kb + 4 * g4 + v;
          if (!(key < S && (!CAUSAL || key <= qrow))) sc[kb][v] = -INFINITY;
        }
    }
    float mx = sc[0][0];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int v = 0; v < 4; ++v) mx = fmaxf(mx, sc[kb][v]);
    const float ms = rows_max(mx) * qk_scale;  // the tile's maximum exponent (-inf: none visible)
    if (__builtin_amdgcn_ballot_w64(ms > m_ref + LAZY)) {
      const float m_new = fmaxf(m_ref, ms);
      const float corr = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_ref - m_new);
      m_ref = m_new;
      l_run *= corr;
#pragma unroll
      for (int b = 0; b < DB; ++b) o[b] *= corr;
    }
    // A query that has seen no visible key yet keeps a zero output.
    const float m_use = m_ref == -INFINITY ? 0.0f : m_ref;
    float psum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        sc[kb][v] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][v], qk_scale, -m_use));
        psum += sc[kb][v];
      }
    l_run += psum;
    // O^T [dh x 16 queries] += V^T P^T over 2 steps of 32 keys.
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const f32x4 a = sc[2 * ks], b2 = sc[2 * ks + 1];
      const bf16x8 pf = {to_bf16(a[0]), to_bf16(a[1]), to_bf16(a[2]), to_bf16(a[3]),
                         to_bf16(b2[0]), to_bf16(b2[1]), to_bf16(b2[2]), to_bf16(b2[3])};
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        // Lane j of the 16-lane group g4 addresses key row base + j / 4 and
        // the 4 dh columns 16 b + 4 (j % 4); it receives dh column 16 b + j
        // of those 4 rows.  Half 0: keys 32 ks + 4 g4 + 0..3, half 1: 16 more.
        s16x4 hv[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int r = 32 * ks + 16 * hh + 4 * g4 + (l16 >> 2);
          const int col = 16 * b + 4 * (l16 & 3);
          const int off = r * (DH * 2) + (((col >> 3) ^ swz_v<DH>(r)) << 4) + ((col & 4) << 1);
          hv[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(vt + off));
        }
        const s16x8 va = {hv[0][0], hv[0][1], hv[0][2], hv[0][3],
                          hv[1][0], hv[1][1], hv[1][2], hv[1][3]};
        o[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va), pf, o[b],
                                                       0, 0, 0);
      }
    }
  };

  // Software pipeline: the key stream runs one tile ahead of the value
  // stream, so that while a wave exponentiates item it's scores the MFMA
  // pipe computes item it+1's.  Buffers: K(it) and V(it) both live in buffer
  // it % 2.  Prologue: K(0), the first scores, then V(0) and K(1).
  f32x4 sc[4], sn[4];
  if (my_n > 0) {
    const int b0 = tile_blk(0), b1 = tile_blk(my_n - 1);
    load_q(qf, b0);
    if (b1 != b0) load_q(qf2, b1);
    qblk = b0;
    issue(0, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
  wg_barrier();
  if (my_n > 0) {
    scores(smem[grp][0][0], sc);
    issue(0, 0, 1);
    if (my_n > 1) issue(1, 1, 0);
  }
  // One iteration; the score registers alternate between sc and sn (the loop
  // below is unrolled by two) instead of being copied.
  auto body = [&](int it, f32x4(&sc)[4], f32x4(&sn)[4]) {
    // V(it) and K(it+1) have landed (this wave's loads; after the barrier,
    // every wave's), and every wave is done with K(it) and V(it-1).
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
    wg_barrier();
    if (it >= my_n) return;
    if (it + 2 < my_n) issue(it + 2, it & 1, 0);
    if (it + 1 < my_n) {
      issue(it + 1, (it + 1) & 1, 1);
      const int nblk1 = tile_blk(it + 1);
      if (nblk1 != qblk) {
#pragma unroll
        for (int s = 0; s < DS; ++s) qf[s] = qf2[s];
        qblk = nblk1;
      }
      scores(smem[grp][(it + 1) & 1][0], sn);
    }
    const int blk = tile_blk(it);
    if (blk != cur) {
      if (cur >= 0) finish_block(cur);
#pragma unroll
      for (int b = 0; b < DB; ++b) o[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      m_ref = -INFINITY;
      l_run = 0.0f;
      cur = blk;
    }
    softmax_pv(sc, smem[grp][it & 1][1], blk, tile_k0(it));
  };
  for (int it = 0; it < half; it += 2) {
    body(it, sc, sn);
    if (it + 1 < half) body(it + 1, sn, sc);
  }
  // No tile load may still be writing LDS when it is reused below or by the
  // next workgroup.
  __builtin_amdgcn_s_waitcnt(wait_vm(0));

  if (split) {
    // Both groups end on the shared block.  Group 0 leaves its state in LDS
    // (lane-indexed, so each lane of group 1's wave gw reads its own
    // counterpart); group 1 merges it into its own and writes the output.
    f32x4 *po = (f32x4 *)&smem[0][0][0][0] + gw * DB * 64 + lane;
    float *pm = (float *)&smem[0][0][0][0] + 4 * 4 * DB * 64 + (gw * 64 + lane) * 2;
    wg_barrier();  // every wave's tile reads are done
    if (grp == 0) {
#pragma unroll
      for (int b = 0; b < DB; ++b) po[b * 64] = o[b];
      pm[0] = m_ref;
      pm[1] = l_run;
    }
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
    wg_barrier();
    if (grp == 1) {
      const float m0 = pm[0], l0 = pm[1];
      const float m = fmaxf(m_ref, m0);
      const float c1 = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_ref - m);
      const float c0 = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m0 - m);
#pragma unroll
      for (int b = 0; b < DB; ++b) o[b] = o[b] * c1 + po[b * 64] * c0;
      l_run = l_run * c1 + l0 * c0;
      finish_block(cur);
    }
  } else if (cur >= 0) {
    finish_block(cur);
  }
}

template <int DH, bool CAUSAL, int HPW>
hipError_t launch_dh(const AttnArgs &a, hipStream_t s) {
  constexpr int QB = 64 / HPW;
  const int64_t nblk = (a.S + QB - 1) / QB;
  const int64_t wgs = a.nseq * (a.Hq / HPW) * ((nblk + 1) / 2);
  if (wgs <= 0) return hipSuccess;
  if (wgs > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attention_kernel<DH, CAUSAL, HPW>), dim3((unsigned)wgs), dim3(NGRP * 256),
                     0, s, a);
  return hipGetLastError();
}

// Query heads per workgroup: the largest of 4, 2, 1 that divides the number
// of query heads per key/value head (TPMLP_ATTN_HEADS caps it, for tuning;
// read once per process).
int heads_per_wg(const AttnArgs &a) {
  static const int cap = [] {
    const char *e = getenv("TPMLP_ATTN_HEADS");
    const int v = e ? atoi(e) : 4;
    return v >= 4 ? 4 : v >= 2 ? 2 : 1;
  }();
  const int grp = a.Hq / a.Hkv;
  for (int hpw = cap; hpw > 1; hpw /= 2)
    if (grp % hpw == 0) return hpw;
  return 1;
}

template <int DH, bool CAUSAL>
hipError_t launch_h(const AttnArgs &a, hipStream_t s) {
  switch (heads_per_wg(a)) {
    case 4: return launch_dh<DH, CAUSAL, 4>(a, s);
    case 2: return launch_dh<DH, CAUSAL, 2>(a, s);
    default: return launch_dh<DH, CAUSAL, 1>(a, s);
  }
}

}  // namespace

bool attention_supported(const AttnArgs &a) {
  // Per-lane DMA offsets are 32-bit byte offsets from a tile's base (64 rows);
  // token indices inside a sequence are 32-bit.
  return (a.dh == 64 || a.dh == 128) && a.Hq >= 1 && a.Hkv >= 1 && a.Hq % a.Hkv == 0 &&
         a.S >= 0 && a.S < (int64_t(1) << 30) && a.ldk < (int64_t(1) << 23) &&
         a.ldv < (int64_t(1) << 23);
}

hipError_t launch_attention(const AttnArgs &a, hipStream_t s) {
  if (!attention_supported(a)) return hipErrorInvalidValue;
  if (a.dh == 128) return a.causal ? launch_h<128, true>(a, s) : launch_h<128, false>(a, s);
  return a.causal ? launch_h<64, true>(a, s) : launch_h<64, false>(a, s);
}

}  // namespace tpmlp
