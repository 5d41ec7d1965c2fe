// Attention core of one head shard for gfx950: per query head,
// O = softmax(Q K^T / sqrt(dh)) V over the keys each query sees (causal or
// not), with grouped key/value heads ("Transformer math: tensor parallel",
// section "Attention: parallel across heads": heads never mix, so a GPU runs
// full attention for its own heads with no communication).
//
// One workgroup of 4 waves owns one query head and two blocks of 64 queries,
// j and N-1-j of the N blocks of a sequence, so that under the causal mask
// every workgroup has the same number of key tiles (the blocks near the start
// see few keys, those near the end many).  Each wave owns 16 queries.  Key and
// value tiles of 64 keys go from HBM to LDS by buffer loads that write LDS
// directly, double-buffered, shared by the 4 waves.
//
// The scores are computed transposed, S^T = K Q^T, with
// v_mfma_f32_16x16x32_bf16: K is the A operand (16-byte LDS reads of 8
// consecutive head dimensions), Q^T the B operand (each lane's 8 head
// dimensions of its query, held in registers for the whole loop).  In the
// accumulator layout every lane then holds 4 keys of ONE query, so the
// running maximum, the running sum and the rescaling of the output are
// lane-local, up to a reduction over the 4 lanes that share a query.  The
// output is accumulated transposed too, O^T += V^T P^T: P^T is the B operand
// straight from the score registers (rounded to bf16), and V^T the A operand,
// read from the [key][dh] tile with the transposing LDS read; the MFMA's
// k-index runs over the keys in the order the score registers hold them
// (keys 4g..4g+3 and 16+4g..16+4g+3 for lane group g), which both operands
// follow, so the sum is unchanged.  The softmax works in base 2: scores are
// scaled by log2(e)/sqrt(dh) and exponentiated with exp2.
#include "device_common.hpp"
#include "kernels.h"
#include "lds_dma.hpp"

namespace tpmlp {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

constexpr int QB = 64;     // queries per block (4 waves x 16)
constexpr int KT = 64;     // keys per tile
constexpr int NWAVE = 4;

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

template <int DH, bool CAUSAL>
__global__ __launch_bounds__(NWAVE * 64, 2) void attention_kernel(AttnArgs p) {
  constexpr int UNITS = DH / 8;                 // 16-byte units per tile row
  constexpr int TILE = KT * DH * 2;             // bytes of one K (or V) tile
  constexpr int LOADS = TILE / 1024 / NWAVE;    // 1 KiB loads per wave per tile
  constexpr int ROWS_PER_LOAD = 1024 / (DH * 2);
  constexpr int DS = DH / 32;                   // 32-dh MFMA steps of the scores
  constexpr int DB = DH / 16;                   // 16-dh output blocks
  __shared__ __attribute__((aligned(1024))) char smem[2][2][TILE];  // [buffer][K or V]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, l16 = lane & 15;
  const int64_t nblk = (p.S + QB - 1) / QB;
  const int64_t npair = (nblk + 1) / 2;
  const int64_t pair = blockIdx.x % npair;
  const int64_t h = (blockIdx.x / npair) % p.Hq;
  const int64_t seq = blockIdx.x / (npair * p.Hq);
  const int64_t c = h / (p.Hq / p.Hkv);        // key/value head
  const bf16 *Qs = (const bf16 *)p.Q + seq * p.S * p.ldq + h * DH;
  const bf16 *Ks = (const bf16 *)p.K + seq * p.S * p.ldk + c * DH;
  const bf16 *Vs = (const bf16 *)p.V + seq * p.S * p.ldv + c * DH;
  bf16 *Os = (bf16 *)p.O + seq * p.S * p.ldo + h * DH;
  const float qk_scale = p.scale_log2;

  // Per-lane DMA offsets inside a tile: load j of wave w fills rows
  // (LOADS w + j) * ROWS_PER_LOAD + lane / UNITS; physical unit lane % UNITS.
  int ld_row[LOADS], ld_ku[LOADS], ld_vu[LOADS];
#pragma unroll
  for (int j = 0; j < LOADS; ++j) {
    const int r = (LOADS * wave + j) * ROWS_PER_LOAD + lane / UNITS;
    ld_row[j] = r;
    ld_ku[j] = (lane % UNITS) ^ swz_k<DH>(r);
    ld_vu[j] = (lane % UNITS) ^ swz_v<DH>(r);
  }
  auto issue_tile = [&](int64_t k0, int buf) {
    const i32x4 rk = rsrc(Ks + k0 * p.ldk), rv = rsrc(Vs + k0 * p.ldv);
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const bool live = k0 + ld_row[j] < p.S;
      dma16(rk, smem[buf][0] + (LOADS * wave + j) * 1024,
            live ? (uint32_t)((ld_row[j] * p.ldk + 8 * ld_ku[j]) * 2) : OOB);
      dma16(rv, smem[buf][1] + (LOADS * wave + j) * 1024,
            live ? (uint32_t)((ld_row[j] * p.ldv + 8 * ld_vu[j]) * 2) : OOB);
    }
  };

  for (int part = 0; part < 2; ++part) {
    const int64_t blk = part == 0 ? pair : nblk - 1 - pair;
    if (part == 1 && blk == pair) break;  // odd block count: the middle block once
    const int64_t q0 = blk * QB;
    const int64_t qrow = q0 + 16 * wave + l16;  // this lane's query (B-operand column)
    // Q^T fragments: 8 consecutive dh of the lane's query per 32-dh step.
    bf16x8 qf[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      if (qrow < p.S)
        qf[s] = *(const bf16x8 *)(Qs + qrow * p.ldq + 32 * s + 8 * g4);
      else
        qf[s] = bf16x8{};
    }
    const int64_t kend = CAUSAL ? (q0 + QB < p.S ? q0 + QB : p.S) : p.S;
    const int ntiles = (int)((kend + KT - 1) / KT);
    f32x4 o[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) o[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY, l_run = 0.0f;

    // Every wave's reads of the previous block's last tiles are done before
    // its buffers are refilled.
    wg_barrier();
    issue_tile(0, 0);
    for (int t = 0; t < ntiles; ++t) {
      const int buf = t & 1;
      const int64_t k0 = (int64_t)t * KT;
      // This wave's loads of tile t have landed; after the barrier every
      // wave's have, and every wave is done reading tile t-1's buffer.
      __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
      wg_barrier();
      if (t + 1 < ntiles) issue_tile(k0 + KT, buf ^ 1);
      const char *kt = smem[buf][0];
      const char *vt = smem[buf][1];

      // ---- scores S^T [64 keys x 16 queries] as 4 blocks of 16 keys ----------
      f32x4 sc[4];
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
      // ---- online softmax (base 2) over the lane's 16 keys of its query -----
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int64_t key = k0 + 16 * kb + 4 * g4 + v;
          const bool vis = key < p.S && (!CAUSAL || key <= qrow);
          const float x = vis ? sc[kb][v] * qk_scale : -INFINITY;
          sc[kb][v] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      // A query that has seen no visible key yet keeps a zero output.
      const float m_use = m_new == -INFINITY ? 0.0f : m_new;
      const float corr = exp2f(m_run - m_use);
      m_run = m_new;
      float psum = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          sc[kb][v] = exp2f(sc[kb][v] - m_use);
          psum += sc[kb][v];
        }
      l_run = l_run * corr + psum;
#pragma unroll
      for (int b = 0; b < DB; ++b) o[b] *= corr;

      // ---- O^T [dh x 16 queries] += V^T P^T over 2 steps of 32 keys ------------
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
    }
    // No tile load may still be writing LDS when the buffers are reused.
    __builtin_amdgcn_s_waitcnt(wait_vm(0));

    // ---- O = O^T / l: lane holds dh rows 16 b + 4 g4 + v of its query ---------
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    if (qrow < p.S) {
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        const bf16x4 w = {to_bf16(o[b][0] * inv), to_bf16(o[b][1] * inv), to_bf16(o[b][2] * inv),
                          to_bf16(o[b][3] * inv)};
        *(bf16x4 *)(Os + qrow * p.ldo + 16 * b + 4 * g4) = w;
      }
    }
  }
}

template <int DH, bool CAUSAL>
hipError_t launch_dh(const AttnArgs &a, hipStream_t s) {
  const int64_t nblk = (a.S + QB - 1) / QB;
  const int64_t wgs = a.nseq * a.Hq * ((nblk + 1) / 2);
  if (wgs <= 0) return hipSuccess;
  if (wgs > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attention_kernel<DH, CAUSAL>), dim3((unsigned)wgs), dim3(NWAVE * 64), 0, s,
                     a);
  return hipGetLastError();
}

}  // namespace

bool attention_supported(const AttnArgs &a) {
  // Per-lane DMA offsets are 32-bit byte offsets from a tile's base (64 rows).
  return (a.dh == 64 || a.dh == 128) && a.Hq >= 1 && a.Hkv >= 1 && a.Hq % a.Hkv == 0 &&
         a.ldk < (int64_t(1) << 23) && a.ldv < (int64_t(1) << 23);
}

hipError_t launch_attention(const AttnArgs &a, hipStream_t s) {
  if (!attention_supported(a)) return hipErrorInvalidValue;
  if (a.dh == 128)
    return a.causal ? launch_dh<128, true>(a, s) : launch_dh<128, false>(a, s);
  return a.causal ? launch_dh<64, true>(a, s) : launch_dh<64, false>(a, s);
}

}  // namespace tpmlp
