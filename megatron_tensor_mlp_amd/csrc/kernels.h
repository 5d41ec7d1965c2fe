// Host-side launch interface of the gfx950 kernels (internal to libtpmlp).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tpmlp {

// What a GEMM does with its fp32 accumulator tile.
enum Epilogue : int {
  EPI_ACT = 0,          // C = act(acc + bias) in the element type  (column step, GeLU/ReLU/none)
  EPI_SWIGLU = 1,       // C = SiLU(acc_gate) * acc_up              (column step, SwiGLU)
  EPI_F32 = 2,          // C = acc, fp32                           (row step partial)
  EPI_F32_ACC = 3,      // C = C + acc, fp32                       (second term of a gradient)
  EPI_ACT_SAVE = 4,     // EPI_ACT, and C2 = acc + bias            (pre-activation kept for
                        //                                          the backward pass)
  EPI_SWIGLU_SAVE = 5,  // EPI_SWIGLU, and C2 = [gate | up]        (columns [0,N) and [N,2N))
  EPI_DACT = 6,         // C = acc * act'(aux)                     (hidden gradient)
  EPI_DSWIGLU = 7,      // C = [acc * up * SiLU'(gate) | acc * SiLU(gate)], aux = [gate | up]
};

// Operand layouts.  A GEMM multiplies A [M,K] by B [K,N]; either operand may
// be stored as its transpose (the backward pass multiplies by transposed
// weights and activations without copying them).
enum Layout : int {
  LAY_NN = 0,  // A row-major [M,K] (k contiguous), B row-major [K,N] (n contiguous)
  LAY_NT = 1,  // B stored as B^T [N,K] (k contiguous; ldb between its rows)
  LAY_TN = 2,  // A stored as A^T [K,M] (m contiguous; lda between its rows)
};

// Column map: output column c of a GEMM reads weight (and bias) column
// c - seg_start[s] + seg_src[s], s the last segment with seg_start[s] <= c.
// With nseg = 0 the map is the identity.  The fused QKV projection of one
// head shard uses three segments (its query, key and value heads).
constexpr int kMaxSegs = 3;

// C[M,N] = epilogue(A[M,K] * B[K,N]) for `groups` independent problems that
// share M, N, K and leading dimensions; problem g uses base pointers offset by
// g * s* elements (the simulated-p grouped launch).  bf16 operands.
struct GemmArgs {
  const void *A;
  int64_t lda;
  const void *B;   // gate matrix for SwiGLU
  int64_t ldb;
  const void *B2;  // up matrix (SwiGLU only)
  int64_t ldb2;
  const void *bias;  // [N] or null (EPI_ACT only)
  void *C;
  int64_t ldc;
  int64_t M, N, K;
  int epi, act;
  int groups;
  int64_t sA, sB, sB2, sBias, sC;
  int nseg;  // column map (EPI_ACT only; 0 = identity)
  int64_t seg_start[kMaxSegs], seg_src[kMaxSegs];
  int lay;          // Layout (LAY_NN unless set)
  void *C2;         // second output (EPI_ACT_SAVE, EPI_SWIGLU_SAVE), element type
  int64_t ldc2;
  const void *aux;  // saved pre-activation (EPI_DACT, EPI_DSWIGLU), element type
  int64_t ldaux;
  // LAY_NT only: B^T rows are the concatenation along k of B^T [N, ksplit]
  // and B2^T [N, K - ksplit] (both with leading dimension ldb), so that
  // A [M, K] times them sums two products in one GEMM; 0 = off.  ksplit is a
  // multiple of 32 (a k-step never straddles the two).
  int64_t ksplit;
  // Tiled path: k-ranges per output tile (split-K), 0 = the launcher's choice
  // (tiled_splitk), 1 = none.  Split tiles meet in the workspace passed to
  // the launch (the shared layout: the counter area, then the partials).
  int splitk;
};

// Weight / bias column read for output column c.
__host__ __device__ inline int64_t src_col(const GemmArgs &p, int64_t c) {
  int64_t base = 0;
  for (int s = 0; s < kMaxSegs; ++s)
    if (s < p.nseg && c >= p.seg_start[s]) base = p.seg_src[s] - p.seg_start[s];
  return c + base;
}

// Large-T path: MFMA tiles staged through LDS (every epilogue and layout).
// _supported: the shape fits the kernels' 32-bit buffer offsets.
// tiled_splitk: the k-ranges per tile the launch uses (a.splitk, or for 0
// the launcher's choice: more than one only for plain layouts with the
// forward epilogues, at most 120 tiles of 256 rows, and k of 1536 or more);
// tiled_workspace_bytes: the workspace that needs (0 without split-K).
bool gemm_bf16_tiled_supported(const GemmArgs &a);
int tiled_splitk(const GemmArgs &a);
size_t tiled_workspace_bytes(const GemmArgs &a);
hipError_t launch_gemm_bf16_tiled(const GemmArgs &a, void *ws, hipStream_t s);

// Every entry point that takes a workspace lays it out the same way, so that
// one buffer can serve them all: a counter area of kWsCounterBytes (arrival
// counters of the few-token path, zero between calls) and scratch after it
// (overwritten before it is read, never assumed zero).
constexpr int64_t kWsMaxBlocks = 65536;  // few-token column blocks per call
constexpr size_t kWsCounterBytes = kWsMaxBlocks * sizeof(unsigned);

// Library-owned scratch for callers that cannot allocate: a static device
// array of kStaticScratchBytes per GPU in the workspace layout above.  Returns
// its address on the current device, looked up (and its counter area zeroed on
// `stream`) at the first call on that device.
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
hipError_t static_scratch(hipStream_t stream, void **ptr);

// Few-token path (M <= 64): weight-streaming split-K GEMM (LAY_NN; EPI_ACT,
// EPI_SWIGLU and EPI_F32).  `ws` must hold
// decode_workspace_bytes(a) zero-initialised bytes (or 0 bytes if that is 0).
// _supported: 1 <= M <= 64 and the shape fits the kernels' 32-bit buffer
// offsets and the workspace's counter area.
size_t decode_workspace_bytes(const GemmArgs &a);
bool gemm_bf16_decode_supported(const GemmArgs &a);
hipError_t launch_gemm_bf16_decode(const GemmArgs &a, void *ws, hipStream_t s);

// MFMA throughput / shader-clock calibration (measurement aid).
hipError_t launch_calib_mfma(int gaussian, int64_t iters, uint64_t *stats, int nwg,
                             hipStream_t s);
// Streaming-read calibration: nwg workgroups read `bytes` (a multiple of 16)
// from `buf` once (measurement aid).
hipError_t launch_calib_hbm_read(const void *buf, int64_t bytes, uint32_t *sink, int nwg,
                                 hipStream_t s);

// Attention core of one head shard (bf16): O = softmax(Q K^T / sqrt(dh)) V per
// query head h, key/value head h / (Hq / Hkv); nseq sequences of S tokens.
struct AttnArgs {
  const void *Q, *K, *V;  // [T, Hq dh], [T, Hkv dh], [T, Hkv dh] (head-major columns)
  void *O;                // [T, Hq dh]
  int64_t ldq, ldk, ldv, ldo;
  int64_t nseq, S;
  int Hq, Hkv, dh, causal;
  float scale_log2;       // log2(e) / sqrt(dh)
};
bool attention_supported(const AttnArgs &a);
hipError_t launch_attention(const AttnArgs &a, hipStream_t s);

// fp32 path (correctness-first): one output per thread, k ascending.
hipError_t launch_gemm_f32(const GemmArgs &a, hipStream_t s);

// out[j] = sum over rows t of H[t, j] (fp32), rows ascending within chunks of
// 64, chunks ascending; ws holds colsum_workspace_bytes(T, n) bytes of scratch.
size_t colsum_workspace_bytes(int64_t T, int64_t n);
hipError_t launch_colsum(bool bf16_in, const void *H, int64_t ldh, int64_t T, int64_t n, float *ws,
                         float *out, hipStream_t s);

// Z = ((P0 + P1) + ...) + P_{p-1} (+ b2), fp32.
constexpr int kMaxParts = 64;
struct PartSumArgs {
  const float *parts[kMaxParts];
  int p;
  int64_t T, d, ldp, ldz;
  const float *b2;
  float *Z;
};
hipError_t launch_partial_sum(const PartSumArgs &a, hipStream_t s);

// Row step of a transformer block: x = (((parts[0] + ...) + bias) + R) in
// fp32 (absent terms skipped), written to X if given, and LayerNorm(x) in
// bf16 to A if gamma is given.  One row per workgroup, held in registers.
constexpr int64_t kRowNormMaxD = 16384;
struct RowNormArgs {
  const float *parts[kMaxParts];
  int p;
  int64_t T, d, ldp;
  const float *bias;
  const float *R;
  int64_t ldr;
  float *X;
  int64_t ldx;
  const float *gamma, *beta;
  float eps;
  void *A;
  int64_t lda;
};
hipError_t launch_residual_ln(const RowNormArgs &a, hipStream_t s);

}  // namespace tpmlp
