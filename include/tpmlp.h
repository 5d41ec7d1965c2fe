/*
 * tpmlp.h -- C ABI of one GPU's shard of a tensor-parallel transformer MLP,
 * for AMD Instinct MI355X (gfx950).
 *
 * The method (Megatron-style tensor parallelism of the feed-forward block):
 *   Y_i = act(X A_i + b1_i)           column-parallel linear, local activation
 *   Z_i = Y_i B_i                     row-parallel linear, full-shape partial
 *   Z   = Z_0 + Z_1 + ... + Z_{p-1}   the reduction (an all-reduce across GPUs;
 *                                     here an on-device sum of p partials)
 * with X [T,d] replicated on every shard, A = W1 [d,k] split by columns,
 * B = W2 [k,d] split by rows, and shard i of p owning hidden units
 * [i*k/p, (i+1)*k/p).  Sources: "Transformer math: tensor parallel"
 * (aicassindra.com), sections "Column-parallel: split the weight by output
 * columns", "Row-parallel: split the weight by input rows" and "The MLP block:
 * column then row, one all-reduce"; "Tensor Parallelism Explained"
 * (initnode.dev), section 1 (equations for Y_i, Z_i and Z) and section 2.B (the
 * SwiGLU variant); the Day 41 post (skandtandon.pages.dev), sections
 * "Simulating column parallel linear", "Simulating row parallel linear" and
 * "Pairing them: the Megatron-LM MLP".
 *
 * Conventions for every entry point:
 *   - Matrices are row-major; a leading dimension (ld*) is the distance in
 *     elements between consecutive rows and must be >= the row width.
 *   - Weights are passed as the FULL logical matrices plus (i, p); the library
 *     takes the shard's column block of W1/Wu/b1 and row block of W2 itself.
 *     A GPU that stores only its compact shard passes it with k = k/p, i = 0,
 *     p = 1 (a column block of a [d,k] matrix is itself a [d,k/p] matrix).
 *   - i is 0-based, 0 <= i < p, 1 <= p <= 64, and k must be divisible by p
 *     ("Tensor Parallelism Explained", section 4: a degree that does not divide
 *     the sharded dimension is a startup error).
 *   - Element types: TP_BF16 means bf16 X, weights, bias and hidden Y with fp32
 *     accumulation; TP_F32 means fp32 throughout.  Partials Z_i and the reduced
 *     Z are always fp32.
 *   - Alignment: every data pointer must be 16-byte aligned, and d, k/p and
 *     every leading dimension must be a multiple of 8 elements (bf16) or
 *     4 elements (fp32); otherwise TP_ERR_MISALIGNED.
 *   - Range (bf16): the kernels address memory with 32-bit offsets, so every
 *     leading dimension must be below 2^23 elements (ldx below 2^21 when
 *     T > 64), and with T <= 64 the output width (k/p, or d) at most 8388608
 *     columns; otherwise TP_ERR_BAD_SHAPE.
 *   - T = 0 is valid and launches nothing; the token-sized buffers (X, Y, Z,
 *     the partials) may then be NULL.
 *   - Memory: all tensors are device memory owned by the caller.  The library
 *     allocates nothing and keeps no pointer after a call returns.  Some shapes
 *     need a caller-provided workspace (see tp_workspace_bytes).
 *   - Streams: `stream` is a hipStream_t (NULL = the default stream).  Work is
 *     enqueued on it and the call returns without waiting; inputs must stay
 *     alive, and outputs must not be read, until the stream reaches the work.
 *   - Errors: arguments are checked on the host before anything is launched.
 *     On any status other than TP_OK nothing was launched and no output was
 *     touched; tp_last_error_message() gives a detail string (per thread).
 *     TP_ERR_HIP means a launch failed; faults during execution surface at the
 *     caller's next synchronisation of the stream.
 *   - Calls on different streams that share a workspace buffer race.
 */
#ifndef TPMLP_H
#define TPMLP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TPMLP_ABI_VERSION 6
#define TP_MAX_SHARDS 64

typedef enum {
  TP_OK = 0,
  TP_ERR_NULL_POINTER = 1, /* a required pointer is NULL                         */
  TP_ERR_BAD_SHAPE = 2,    /* T < 0, d < 1, k < 1, or an ld below the row width  */
  TP_ERR_NOT_DIVISIBLE = 3,/* k % p != 0 (head counts % p != 0 for the QKV step) */
  TP_ERR_BAD_SHARD = 4,    /* i outside [0,p), p < 1 or p > TP_MAX_SHARDS         */
  TP_ERR_MISALIGNED = 5,   /* pointer not 16-byte aligned or width/ld not a
                              multiple of 8 (bf16) / 4 (fp32) elements            */
  TP_ERR_BAD_DTYPE = 6,    /* unknown tp_dtype                                    */
  TP_ERR_BAD_ACT = 7,      /* unknown tp_act, or a bias given with TP_ACT_SWIGLU  */
  TP_ERR_WORKSPACE = 8,    /* workspace missing or smaller than required          */
  TP_ERR_HIP = 9           /* a HIP launch failed                                 */
} tp_status;

typedef enum { TP_F32 = 0, TP_BF16 = 1 } tp_dtype;

/* Local activation of the column step.  GeLU is named by every page without a
 * formula; both published forms are offered: tanh form 0.5x(1+tanh(sqrt(2/pi)
 * (x+0.044715x^3))) and erf form 0.5x(1+erf(x/sqrt2)).  ReLU is the Day 41
 * post's simplification.  TP_ACT_SWIGLU is Swish(X Wg_i) * (X Wu_i) with the
 * Swish slope 1, i.e. SiLU(x) = x/(1+exp(-x)) ("Tensor Parallelism Explained",
 * section 2.B); W1 is then the gate matrix and Wu the up matrix. */
typedef enum {
  TP_ACT_NONE = 0,
  TP_ACT_RELU = 1,
  TP_ACT_GELU_TANH = 2,
  TP_ACT_GELU_ERF = 3,
  TP_ACT_SWIGLU = 4
} tp_act;

/*
 * Column-parallel step of shard i of p (the first linear of the MLP plus its
 * local activation).  With s = k/p and c0 = i*s:
 *   Y[t, j] = act( sum_c X[t,c] * W1[c, c0+j]  +  b1[c0+j] )        (0 <= j < s)
 * or, for TP_ACT_SWIGLU,
 *   Y[t, j] = SiLU( sum_c X[t,c] * W1[c, c0+j] ) * ( sum_c X[t,c] * Wu[c, c0+j] )
 * Source: "Transformer math: tensor parallel", section "Column-parallel: split
 * the weight by output columns" (Y_i = X A_i); the bias slice follows the Day
 * 41 post, "Simulating column parallel linear".
 *   X  [T, d], ldx     input, dtype dt (replicated on every shard)
 *   W1 [d, k], ldw1    full first weight (gate for SwiGLU), dtype dt
 *   Wu [d, k], ldwu    full up weight, SwiGLU only (else NULL, ldwu ignored)
 *   b1 [k] or NULL     full column bias, dtype dt; must be NULL for SwiGLU
 *   Y  [T, s], ldy     output hidden shard, dtype dt, overwritten
 * fp32 accumulation; the activation is applied in fp32 and Y is rounded once
 * (to nearest even) to dt.
 */
tp_status tp_col_linear(tp_dtype dt, tp_act act, int64_t T, int64_t d, int64_t k, int32_t i,
                        int32_t p, const void *X, int64_t ldx, const void *W1, int64_t ldw1,
                        const void *Wu, int64_t ldwu, const void *b1, void *Y, int64_t ldy,
                        void *ws, size_t ws_bytes, void *stream);

/*
 * Row-parallel step of shard i of p (the second linear, without its bias):
 *   Z[t, n] = sum_j Y[t, j] * W2[c0+j, n]                         (0 <= n < d)
 * Source: "Transformer math: tensor parallel", section "Row-parallel: split
 * the weight by input rows" (Z_i = Y_i B_i, a full-shape partial); "Tensor
 * Parallelism Explained", section 1.B.
 *   Y  [T, s], ldy     hidden shard, dtype dt
 *   W2 [k, d], ldw2    full second weight, dtype dt
 *   Z  [T, d], ldz     fp32 partial, overwritten; the row bias is NOT added
 *                      here (it is added once after the reduction)
 */
tp_status tp_row_linear(tp_dtype dt, int64_t T, int64_t d, int64_t k, int32_t i, int32_t p,
                        const void *Y, int64_t ldy, const void *W2, int64_t ldw2, float *Z,
                        int64_t ldz, void *ws, size_t ws_bytes, void *stream);

/*
 * The whole shard: tp_col_linear into the caller's Y, then tp_row_linear from
 * it into Z, on one stream.  Y is an output too (the hidden shard, written once
 * in dt).  Source: "Transformer math: tensor parallel", section "The MLP block:
 * column then row, one all-reduce"; Day 41 post, "Pairing them: the
 * Megatron-LM MLP".
 */
tp_status tp_mlp_shard(tp_dtype dt, tp_act act, int64_t T, int64_t d, int64_t k, int32_t i,
                       int32_t p, const void *X, int64_t ldx, const void *W1, int64_t ldw1,
                       const void *Wu, int64_t ldwu, const void *b1, const void *W2,
                       int64_t ldw2, void *Y, int64_t ldy, float *Z, int64_t ldz, void *ws,
                       size_t ws_bytes, void *stream);

/*
 * tp_mlp_shard for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments (without ws/ws_bytes), results and checks
 * as tp_mlp_shard, except that GEMMs with more than 64 tokens never split K
 * here: where tp_mlp_shard splits one (few output tiles, long K; see
 * tp_workspace_bytes) the fp32 sums are taken in another order, and the two
 * results agree within the bf16 tolerance rather than bit for bit.  The scratch
 * the few-token (T <= 64, bf16) path needs -- its
 * arrival counters and split-K partials -- lives in a library-owned static
 * device array of TP_STATIC_SCRATCH_BYTES on each GPU the library runs on,
 * held until the process ends; its address is looked up, and its counter area
 * cleared by a fill kernel on `stream`, at the first call on each device.  The
 * call allocates nothing (no hipMalloc, hipFree or allocating library call).
 *   - Sizes whose few-token scratch need exceeds TP_STATIC_SCRATCH_BYTES (the
 *     need tp_workspace_bytes reports for T <= 64) return TP_ERR_WORKSPACE,
 *     with nothing launched.
 *   - Every call on one GPU shares that GPU's array, whose content carries
 *     over from call to call (each call leaves the counters zero again):
 *     calls that overlap on one GPU -- on different streams, or from several
 *     host threads without ordering -- race and give wrong results.
 */
#define TP_STATIC_SCRATCH_BYTES ((size_t)16 << 20)
tp_status tp_mlp_shard_noalloc(tp_dtype dt, tp_act act, int64_t T, int64_t d, int64_t k, int32_t i,
                               int32_t p, const void *X, int64_t ldx, const void *W1,
                               int64_t ldw1, const void *Wu, int64_t ldwu, const void *b1,
                               const void *W2, int64_t ldw2, void *Y, int64_t ldy, float *Z,
                               int64_t ldz, void *stream);

/*
 * The reduction of p partials (what the all-reduce computes), on one device:
 *   Z = ((parts[0] + parts[1]) + ...) + parts[p-1]   (+ b2, added once)
 * in fp32, element by element, shard 0 first.  Source: Day 41 post,
 * "Simulating row parallel linear" (sum of the partials, then the bias);
 * "Building GPT from Scratch, Part 9", "Implementation Sketch" (the row bias is
 * added after the all-reduce).
 *   parts  HOST array of p device pointers, each to an fp32 [T, d] matrix
 *          with leading dimension ldp
 *   b2     fp32 [d] or NULL
 *   Z      fp32 [T, d], ldz, overwritten.  Z may be exactly parts[0] (in
 *          place); any other overlap with an input is undefined.
 */
tp_status tp_partial_sum(int64_t T, int64_t d, int32_t p, const float *const *parts, int64_t ldp,
                         const float *b2, float *Z, int64_t ldz, void *stream);

/*
 * Simulated-p mode: all p shards of the MLP on this one device, then the
 * on-device reduction.  Equivalent to tp_mlp_shard for i = 0..p-1 followed by
 * tp_partial_sum, but the shards of each step run as one grouped launch.
 * It lets one GPU check the identity sum_i Z_i = act(X W1) W2 ("Tensor
 * Parallelism Explained", section 1.B, the equation for Z).
 *   Y      p consecutive [T, k/p] blocks (dense), dtype dt: Y_0, Y_1, ...
 *   Zp     p consecutive fp32 [T, d] blocks (dense): the partials Z_0, ...
 *   b2     fp32 [d] or NULL (added once, after the sum)
 *   Z      fp32 [T, d], ldz: the reduced output
 */
tp_status tp_mlp_simulated(tp_dtype dt, tp_act act, int64_t T, int64_t d, int64_t k, int32_t p,
                           const void *X, int64_t ldx, const void *W1, int64_t ldw1,
                           const void *Wu, int64_t ldwu, const void *b1, const void *W2,
                           int64_t ldw2, const float *b2, void *Y, float *Zp, float *Z,
                           int64_t ldz, void *ws, size_t ws_bytes, void *stream);

/*
 * Bytes of workspace that tp_col_linear / tp_row_linear / tp_mlp_shard /
 * tp_mlp_simulated need for these sizes (0 if none).  The workspace holds
 * arrival counters (the first 256 KiB) and split-K partial sums (after them):
 * those of the few-token (T <= 64) path, and with more tokens those of a
 * GEMM with too few output tiles to fill the device (at most 120 tiles of 256
 * rows) and K of 1536 or more, whose k-range is split over 2 to 8 workgroups
 * per tile (at most 60 MiB of partials).  With more than 64 tokens the
 * workspace is optional: given none (NULL), or fewer bytes than this, those
 * GEMMs run unsplit -- slower, and their fp32 sums taken in another order, so
 * the results agree with the split ones within the bf16 tolerance rather than
 * bit for bit.  With 64 or fewer tokens it is required (TP_ERR_WORKSPACE
 * otherwise).  It must be zero-filled before its
 * first use; every call leaves its counters zero again, and no entry point
 * writes anything but zeros to the counter area, so one zeroed buffer can be
 * reused by any later call of any entry point on the same stream.  Returns 0
 * for invalid arguments.
 */
size_t tp_workspace_bytes(tp_dtype dt, tp_act act, int64_t T, int64_t d, int64_t k, int32_t p);

/*
 * Training forward of the column step: tp_col_linear, and in the same launch
 * the pre-activation the backward pass needs,
 *   H[t, j] = sum_c X[t,c] * W1[c, c0+j] + b1[c0+j]                  [T, s]
 * or, for TP_ACT_SWIGLU, H = [G | U] with G = X Wg_i in columns [0, s) and
 * U = X Wu_i in columns [s, 2s)                                      [T, 2s]
 * rounded once to dt like Y.  Always runs the tiled (bf16) or fp32 kernels,
 * whatever T; needs no workspace.
 *   H [T, s] (SwiGLU [T, 2s]), ldh   output, dtype dt, overwritten
 */
tp_status tp_col_linear_train(tp_dtype dt, tp_act act, int64_t T, int64_t d, int64_t k, int32_t i,
                              int32_t p, const void *X, int64_t ldx, const void *W1, int64_t ldw1,
                              const void *Wu, int64_t ldwu, const void *b1, void *Y, int64_t ldy,
                              void *H, int64_t ldh, void *stream);

/*
 * Backward pass of shard i of p, given the gradient dZ of the loss with
 * respect to the reduced output Z = sum_i Z_i.  The reduction's backward is
 * the identity, so every shard receives the same dZ; the row-parallel step's
 * input gradient is local; the column-parallel step's input gradient is one
 * term of a sum over the shards, dX = sum_i dH_i W1_i^T, the all-reduce before
 * the block ("Transformer math: tensor parallel", sections "Column-parallel:
 * split the weight by output columns", "Row-parallel: split the weight by
 * input rows" and "The f and g conjugate operators").  With s = k/p, c0 = i*s:
 *   dY  = dZ W2[c0:c0+s, :]^T                        (not stored)
 *   dH  = dY * act'(H)                               [T, s]   dtype dt
 *         SwiGLU: [dG | dU], dG = dY * U * SiLU'(G), dU = dY * SiLU(G)   [T, 2s]
 *   dXp = dH W1[:, c0:c0+s]^T (+ dU Wu[:, c0:c0+s]^T)    [T, d]  fp32, this
 *         shard's term of dX (sum the p terms with tp_partial_sum)
 *   dW1 = X^T dH (SwiGLU: X^T dG)                    [d, s]   fp32
 *   dWu = X^T dU (SwiGLU only, else NULL)            [d, s]   fp32
 *   db1 = sum over t of dH[t, :]                     [s]      fp32, or NULL
 *         (must be NULL with SwiGLU; needs tp_backward_workspace_bytes)
 *   dW2 = Y^T dZ                                     [s, d]   fp32
 * Inputs (dtype dt): X [T,d]; the full W1, Wu [d,k] and W2 [k,d] as in the
 * forward; H and Y as written by tp_col_linear_train; dZ [T,d].  The
 * activation derivatives are those of the forward's definitions (ReLU'(0) =
 * 0).  Weight-gradient outputs are compact [d, s] / [s, d] matrices,
 * overwritten (not accumulated).  With T = 0 the weight and bias gradients
 * are set to zero and nothing else is touched.  Always runs the tiled (bf16)
 * or fp32 kernels; the operands W2_i^T, W1_i^T, X^T and Y^T are read in place
 * (no transposed copies).
 */
tp_status tp_mlp_shard_backward(tp_dtype dt, tp_act act, int64_t T, int64_t d, int64_t k, int32_t i,
                                int32_t p, const void *X, int64_t ldx, const void *W1, int64_t ldw1,
                                const void *Wu, int64_t ldwu, const void *W2, int64_t ldw2,
                                const void *H, int64_t ldh, const void *Y, int64_t ldy,
                                const void *dZ, int64_t lddz, void *dH, int64_t lddh, float *dXp,
                                int64_t lddx, float *dW1, int64_t lddw1, float *dWu, int64_t lddwu,
                                float *db1, float *dW2, int64_t lddw2, void *ws, size_t ws_bytes,
                                void *stream);

/* Bytes of workspace tp_mlp_shard_backward needs (0 if none): the bias
 * gradient's column sums when with_db1 is non-zero.  The layout is the one
 * tp_workspace_bytes describes (a counter area, then scratch), so one
 * zero-filled buffer of the largest size any call needs serves every entry
 * point on a stream.  Returns 0 for invalid arguments. */
size_t tp_backward_workspace_bytes(tp_dtype dt, tp_act act, int64_t T, int64_t d, int64_t k,
                                   int32_t p, int32_t with_db1);

/*
 * Attention projections of head shard i of p.
 *
 * Multi-head attention splits across GPUs along its heads: shard i owns query
 * heads [i*Hq/p, (i+1)*Hq/p) and key/value heads [i*Hkv/p, (i+1)*Hkv/p), and
 * projects the replicated input X to the queries, keys and values of those
 * heads alone; the QKV projection is thus a column-parallel linear whose
 * column blocks are whole heads ("Transformer math: tensor parallel", section
 * "Attention: parallel across heads"; "Tensor Parallelism Explained", section
 * 2.A; "Building GPT from Scratch, Part 9", section "Splitting the Attention
 * Layer").  With grouped key/value heads (Hkv < Hq) both counts are split p
 * ways ("What is Tensor Parallelism?", Llama 3.1 70B worked example: 64 query
 * and 8 key/value heads give 8 and 1 per GPU at TP = 8).  Hq and Hkv must be
 * divisible by p (TP_ERR_NOT_DIVISIBLE otherwise; "Tensor Parallelism
 * Explained", section 4).  With qw = Hq*dh/p and kw = Hkv*dh/p:
 *   QKV[t, j]           = sum_c X[t,c] Wqkv[c, i*qw + j]                 + b   (j < qw)
 *   QKV[t, qw + j]      = sum_c X[t,c] Wqkv[c, Hq*dh + i*kw + j]         + b   (j < kw)
 *   QKV[t, qw + kw + j] = sum_c X[t,c] Wqkv[c, (Hq+Hkv)*dh + i*kw + j]   + b   (j < kw)
 * (b the same column of bqkv, or 0), in one launch.
 *   X    [T, d], ldx              input, dtype dt (replicated on every shard)
 *   Wqkv [d, (Hq+2*Hkv)*dh], ldw  full packed projection, dtype dt: the query
 *                                 heads' columns, then the key heads', then the
 *                                 value heads'; head h of a block owns its dh
 *                                 columns starting at h*dh
 *   bqkv [(Hq+2*Hkv)*dh] or NULL  full bias, same layout, dtype dt
 *   QKV  [T, qw + 2*kw], ldo      output, dtype dt, overwritten: this shard's
 *                                 query heads, then its key heads, then its value
 *                                 heads (the q | k | v split of the per-GPU
 *                                 projection in the Part 9 module)
 * d and dh must be multiples of 8 (bf16) or 4 (fp32) elements.  fp32
 * accumulation, output rounded once to dt.  A GPU that stores only its own
 * packed [Q_i | K_i | V_i] weight passes it with Hq/p, Hkv/p, i = 0, p = 1.
 *
 * The output projection W_O [Hq*dh, d] is a row-parallel linear over the same
 * head split (its row block of shard i is the rows of the shard's query heads):
 * call tp_row_linear with k = Hq*dh on the shard's attention output
 * [T, Hq*dh/p], and reduce the fp32 partials with tp_partial_sum.
 */
tp_status tp_qkv_linear(tp_dtype dt, int64_t T, int64_t d, int32_t Hq, int32_t Hkv, int64_t dh,
                        int32_t i, int32_t p, const void *X, int64_t ldx, const void *Wqkv,
                        int64_t ldw, const void *bqkv, void *QKV, int64_t ldo, void *ws,
                        size_t ws_bytes, void *stream);

/*
 * Attention core of head shard i, between the QKV projection and W_O (bf16
 * only): for every sequence, query head h and query token t,
 *   O[t, h] = sum_j softmax_j( Q[t, h] . K[j, c] / sqrt(dh) ) V[j, c]
 * over the keys j of t's sequence (j <= t when causal != 0), with
 * c = h / (Hq / Hkv) the key/value head query head h reads.  Heads never mix,
 * so a GPU computes the attention of its own heads with no communication
 * ("Transformer math: tensor parallel", section "Attention: parallel across
 * heads"; the causal form is the GPT module's of "Building GPT from Scratch,
 * Part 9").  Here Hq and Hkv are the shard's own head counts.
 *   T = nseq * S tokens: nseq sequences of S consecutive tokens
 *   Q [T, Hq dh], ldq; K and V [T, Hkv dh], ldk, ldv   (head h in columns
 *     [h dh, (h+1) dh)); the output of tp_qkv_linear is Q = QKV, K = QKV + qw,
 *     V = QKV + qw + kw with ldq = ldk = ldv = its ldo
 *   O [T, Hq dh], ldo   output, overwritten; the input of the W_O row block
 * dh must be 64 or 128 (TP_ERR_BAD_SHAPE otherwise), Hq a multiple of Hkv
 * (TP_ERR_NOT_DIVISIBLE).  fp32 softmax and accumulation; the probabilities
 * enter the second product rounded to bf16.  No workspace.
 */
tp_status tp_attention(tp_dtype dt, int64_t nseq, int64_t S, int32_t Hq, int32_t Hkv, int64_t dh,
                       int32_t causal, const void *Q, int64_t ldq, const void *K, int64_t ldk,
                       const void *V, int64_t ldv, void *O, int64_t ldo, void *stream);

/* Bytes of workspace tp_qkv_linear needs for these sizes (0 if none, or for
 * invalid arguments); the same contract as tp_workspace_bytes. */
size_t tp_qkv_workspace_bytes(tp_dtype dt, int64_t T, int64_t d, int32_t Hq, int32_t Hkv,
                              int64_t dh, int32_t p);

/*
 * Row step of a transformer block ("Building GPT from Scratch, Part 9",
 * section "Communication Pattern per Transformer Block": each half of the
 * block ends in an all-reduce of the row-parallel partials and a residual
 * add, and each half begins with a LayerNorm every GPU applies to the full
 * row).  For every token row t:
 *   x = (((parts[0][t] + parts[1][t]) + ...) + bias) + R[t]
 *       fp32, added left to right in that order; absent terms are skipped
 *       (p = 0: no partials; bias or R NULL), at least one term is present
 *   X[t] = x                                     if X != NULL   (fp32)
 *   A[t] = (x - mean) / sqrt(var + eps) * gamma + beta
 *       if A != NULL (bf16, rounded once), with the mean and the biased
 *       variance over the row's d elements; gamma, beta [d] fp32
 *   T >= 0, 8 <= d <= 16384 and d a multiple of 8; p in [0, TP_MAX_SHARDS];
 *   parts: host array of p device pointers to [T, d] fp32 (ldp); R [T, d]
 *   fp32 (ldr); X [T, d] fp32 (ldx), may alias R or parts[0] (in place);
 *   A [T, d] bf16 (lda), the input of the next half's GEMMs.
 * gamma, beta and A are given together or not at all; eps finite and >= 0.
 * With T = 0 nothing is read or written and the buffers may be NULL.
 * The X it writes equals the same left-to-right fp32 sum bit for bit.
 * Errors as elsewhere (TP_ERR_BAD_SHAPE, TP_ERR_MISALIGNED,
 * TP_ERR_NULL_POINTER, TP_ERR_BAD_SHARD); nothing is launched on error.
 */
tp_status tp_residual_layernorm(int64_t T, int64_t d, int32_t p, const float *const *parts,
                                int64_t ldp, const float *bias, const float *R, int64_t ldr,
                                float *X, int64_t ldx, const float *gamma, const float *beta,
                                float eps, void *A, int64_t lda, void *stream);

/*
 * One pre-LayerNorm transformer block of p tensor-parallel shards, all run on
 * this GPU (bf16 weights and GEMM inputs, fp32 residual stream), in the order
 * of "Building GPT from Scratch, Part 9", section "Communication Pattern per
 * Transformer Block":
 *   A    = LN1(X)
 *   for shard i: QKV_i = A Wqkv[:, heads of i] + bqkv   (as tp_qkv_linear)
 *                O_i   = attention of shard i's heads   (as tp_attention)
 *                P_i   = O_i WO[rows of i's heads, :]   (as tp_row_linear)
 *   X1   = ((P_0 + P_1) + ...) + bO + X                  (reduction #1)
 *   A    = LN2(X1)
 *   for shard i: Z_i = act(A W1_i + b1_i) W2_i (or SwiGLU), as tp_mlp_simulated
 *   Out  = ((Z_0 + Z_1) + ...) + b2 + X1                 (reduction #2)
 * The two sums stand for the two all-reduces of the block; every step runs
 * in this library's kernels (tp_residual_layernorm's for the sums and the
 * LayerNorms).  The p shards' QKV column blocks together are the whole
 * projection and are computed by one launch, the attention core runs over all
 * heads in one launch, and the W_O row blocks and the FFN shards are grouped
 * launches that write one partial per shard; each element is computed as in
 * the shard's own launch.
 *   T = nseq * S tokens (nseq sequences of S; attention causal when causal
 *   != 0); X, Out [T, d] fp32 (ldx, ldout), Out may alias X;
 *   ln1_g, ln1_b, ln2_g, ln2_b [d] fp32; eps as in tp_residual_layernorm;
 *   Wqkv [d, (Hq + 2 Hkv) dh] packed as for tp_qkv_linear (ldwqkv), bqkv
 *   [(Hq + 2 Hkv) dh] or NULL; WO [Hq dh, d] (ldwo), bO [d] fp32 or NULL;
 *   W1 (and Wu for TP_ACT_SWIGLU) [d, k], b1 [k] or NULL (not with SwiGLU),
 *   W2 [k, d], b2 [d] fp32 or NULL.
 * dt must be TP_BF16; dh 64 or 128; Hq, Hkv and k divisible by p and Hq by
 * Hkv (TP_ERR_NOT_DIVISIBLE); 8 <= d <= 16384, a multiple of 8.  Workspace:
 * at least tp_block_workspace_bytes (the shared layout: zeroed counter area,
 * then scratch; it holds A, the QKV projection and attention output of all
 * heads, the p hidden shards and p fp32 [T, d] partials).  Nothing is launched on error.
 */
tp_status tp_block_simulated(tp_dtype dt, tp_act act, int64_t nseq, int64_t S, int64_t d,
                             int32_t Hq, int32_t Hkv, int64_t dh, int64_t k, int32_t p,
                             int32_t causal, float eps, const float *X, int64_t ldx,
                             const float *ln1_g, const float *ln1_b, const void *Wqkv,
                             int64_t ldwqkv, const void *bqkv, const void *WO, int64_t ldwo,
                             const float *bO, const float *ln2_g, const float *ln2_b,
                             const void *W1, int64_t ldw1, const void *Wu, int64_t ldwu,
                             const void *b1, const void *W2, int64_t ldw2, const float *b2,
                             float *Out, int64_t ldout, void *ws, size_t ws_bytes, void *stream);

/* Bytes of workspace tp_block_simulated needs for these sizes (0 for invalid
 * arguments or no tokens). */
size_t tp_block_workspace_bytes(tp_dtype dt, tp_act act, int64_t nseq, int64_t S, int64_t d,
                                int32_t Hq, int32_t Hkv, int64_t dh, int64_t k, int32_t p);

/* Shard bookkeeping on the host: shard i of p of a dimension of size k owns
 * [*c0, *c0 + *s) with s = k/p and c0 = i*s (Day 41 post, "Simulating column
 * parallel linear").  No GPU is touched. */
tp_status tp_shard_bounds(int64_t k, int32_t i, int32_t p, int64_t *c0, int64_t *s);

const char *tp_status_string(tp_status s);
const char *tp_last_error_message(void); /* detail of this thread's last non-OK status */
int32_t tp_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* TPMLP_H */
