/*
 * CPU oracle for one tensor-parallel MLP shard, forward and backward (and the
 * attention projections of one head shard).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain reference that the
 * GPU library is checked against.  Only the test suite, the smoke check and
 * the benchmark's CPU-baseline leg may load it.  It shares no code, header,
 * table or helper with the HIP library, and it includes nothing from it.
 *
 * What it computes (the plain definition, written out):
 *
 *   Shard i of p owns the contiguous block of s = k/p hidden units starting
 *   at c0 = i*s.
 *     - Column-parallel linear: each shard multiplies the full, replicated
 *       input X [T,d] by its own column block of A [d,k] and keeps a [T,s]
 *       slice of the hidden activation ("Transformer math: tensor parallel",
 *       section "Column-parallel: split the weight by output columns";
 *       "Tensor Parallelism Explained", section 1.A).  The column bias is cut
 *       the same way as the columns (Day 41 post, "Simulating column parallel
 *       linear").
 *     - The activation is element-wise, so it is applied to the shard alone
 *       ("Transformer math: tensor parallel", section "The MLP block: column
 *       then row, one all-reduce").  For the gated variant both the gate and
 *       the up projection are column-split the same way and the shard forms
 *       Swish(gate) times up ("Tensor Parallelism Explained", section 2.B).
 *     - Row-parallel linear: the shard multiplies its hidden slice by its row
 *       block of B [k,d] and gets a full-shape [T,d] partial ("Transformer
 *       math: tensor parallel", section "Row-parallel: split the weight by
 *       input rows").
 *     - The reduction adds the p partials element by element, shard 0 first,
 *       then adds the row bias once (Day 41 post, "Simulating row parallel
 *       linear").
 *     - Attention is split the same way along its heads: the QKV projection is
 *       a column-parallel linear whose column blocks are whole heads, and the
 *       output projection is the row-parallel linear above over the head
 *       columns (oracle_qkv_shard_f64 below).
 *     - The attention core between the projections, per head with grouped
 *       key/value heads, causal or not (oracle_attention_f64 below).
 *     - One pre-LayerNorm transformer block (oracle_layernorm_f64 and
 *       oracle_block_f64 below), unsharded: the reference a sharded block is
 *       checked against.
 *     - The backward pass of a shard (oracle_mlp_shard_backward_f64 below):
 *       the row-parallel step's input gradient is local, the column-parallel
 *       step's is one term of a sum over the shards.
 *
 * Every dot product is summed with its index ascending, in the precision of
 * the function (fp64, or fp32 for the *_f32 functions that pin the printed
 * fp32 result of the Day 41 post).  There is no blocking, no reordering and
 * no intermediate rounding.  Rows of the output are spread over OpenMP
 * threads; that does not change any sum.  Build with -ffp-contract=off so
 * that a multiply followed by an add is never fused into one rounding.
 *
 * Activations follow their published definitions; the pages only name them:
 *   GeLU, tanh form: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))
 *                    (Hendrycks and Gimpel, 2016)
 *   GeLU, erf form:  0.5 x (1 + erf(x / sqrt 2))
 *   SiLU (Swish with beta = 1): x / (1 + exp(-x))
 *   ReLU: max(0, x)  (Day 41 post, "Pairing them: the Megatron-LM MLP")
 * They call the host C library (tanh, erf, exp).
 *
 * Matrices are dense row-major with no padding.  All pointers are host
 * memory owned by the caller.  Functions return 0, or -1 on an argument that
 * breaks the shard rule (k not divisible by p, i outside [0,p)).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Activation kinds understood by this oracle (its own numbering). */
#define OR_ACT_NONE 0
#define OR_ACT_RELU 1
#define OR_ACT_GELU_TANH 2
#define OR_ACT_GELU_ERF 3
#define OR_ACT_SWIGLU 4 /* column step: SiLU(gate) * up; scalar helper: SiLU */

static double act_scalar_f64(int kind, double x) {
  switch (kind) {
    case OR_ACT_NONE:
      return x;
    case OR_ACT_RELU:
      return x > 0.0 ? x : 0.0;
    case OR_ACT_GELU_TANH: {
      const double c = sqrt(2.0 / M_PI);
      return 0.5 * x * (1.0 + tanh(c * (x + 0.044715 * x * x * x)));
    }
    case OR_ACT_GELU_ERF:
      return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));
    case OR_ACT_SWIGLU:
      return x / (1.0 + exp(-x));
  }
  return NAN;
}

static float act_scalar_f32(int kind, float x) {
  switch (kind) {
    case OR_ACT_NONE:
      return x;
    case OR_ACT_RELU:
      return x > 0.0f ? x : 0.0f;
    case OR_ACT_GELU_TANH: {
      const float c = (float)sqrt(2.0 / M_PI);
      return 0.5f * x * (1.0f + tanhf(c * (x + 0.044715f * x * x * x)));
    }
    case OR_ACT_GELU_ERF:
      return 0.5f * x * (1.0f + erff(x / sqrtf(2.0f)));
    case OR_ACT_SWIGLU:
      return x / (1.0f + expf(-x));
  }
  return NAN;
}

static int shard_ok(int64_t k, int32_t i, int32_t p) {
  return p >= 1 && i >= 0 && i < p && k % p == 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* y[n] = act(x[n]) for the scalar activations (kind 4 is SiLU here). */
void oracle_activation_f64(int kind, int64_t n, const double *x, double *y) {
  for (int64_t e = 0; e < n; ++e) y[e] = act_scalar_f64(kind, x[e]);
}

/*
 * Column-parallel step of shard i of p, fp64.
 *   X  [T,d]; W1 [d,k] (the full matrix, the gate for SwiGLU); Wu [d,k] (up,
 *   SwiGLU only, else NULL); b1 [k] or NULL (not used with SwiGLU).
 *   Y  [T,k/p] receives act(X W1[:, c0:c0+s] + b1[c0:c0+s]), or
 *   SiLU(X Wg[:, c0:c0+s]) * (X Wu[:, c0:c0+s]).
 */
int oracle_col_shard_f64(int64_t T, int64_t d, int64_t k, int32_t i, int32_t p,
                         const double *X, const double *W1, const double *Wu,
                         const double *b1, int act, double *Y) {
  if (!shard_ok(k, i, p)) return -1;
  if (act == OR_ACT_SWIGLU && Wu == NULL) return -1;
  const int64_t s = k / p, c0 = (int64_t)i * s;
#pragma omp parallel
  {
    double *u = (double *)malloc(sizeof(double) * (size_t)(s > 0 ? s : 1));
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      double *h = Y + t * s;
      for (int64_t j = 0; j < s; ++j) h[j] = 0.0;
      for (int64_t j = 0; j < s; ++j) u[j] = 0.0;
      for (int64_t c = 0; c < d; ++c) {
        const double xv = X[t * d + c];
        const double *w = W1 + c * k + c0;
        for (int64_t j = 0; j < s; ++j) h[j] += xv * w[j];
        if (act == OR_ACT_SWIGLU) {
          const double *wu = Wu + c * k + c0;
          for (int64_t j = 0; j < s; ++j) u[j] += xv * wu[j];
        }
      }
      if (act == OR_ACT_SWIGLU) {
        for (int64_t j = 0; j < s; ++j) h[j] = act_scalar_f64(OR_ACT_SWIGLU, h[j]) * u[j];
      } else {
        for (int64_t j = 0; j < s; ++j) {
          const double v = b1 ? h[j] + b1[c0 + j] : h[j];
          h[j] = act_scalar_f64(act, v);
        }
      }
    }
    free(u);
  }
  return 0;
}

/*
 * Row-parallel step of shard i of p, fp64.
 *   Y [T,k/p] (this shard's hidden slice); W2 [k,d] (the full matrix).
 *   Z [T,d] receives Y W2[c0:c0+s, :], the shard's partial (no bias).
 */
int oracle_row_shard_f64(int64_t T, int64_t d, int64_t k, int32_t i, int32_t p,
                         const double *Y, const double *W2, double *Z) {
  if (!shard_ok(k, i, p)) return -1;
  const int64_t s = k / p, c0 = (int64_t)i * s;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    double *z = Z + t * d;
    for (int64_t n = 0; n < d; ++n) z[n] = 0.0;
    for (int64_t j = 0; j < s; ++j) {
      const double yv = Y[t * s + j];
      const double *w = W2 + (c0 + j) * d;
      for (int64_t n = 0; n < d; ++n) z[n] += yv * w[n];
    }
  }
  return 0;
}

/*
 * The reduction that replaces the all-reduce, fp64:
 *   Z = ((parts[0] + parts[1]) + ...) + parts[p-1], then + b2 (if given).
 *   parts is p consecutive [T,d] blocks.
 */
int oracle_partial_sum_f64(int64_t T, int64_t d, int32_t p, const double *parts,
                           const double *b2, double *Z) {
  if (p < 1) return -1;
  const int64_t n = T * d;
#pragma omp parallel for schedule(static)
  for (int64_t e = 0; e < n; ++e) {
    double acc = parts[e];
    for (int32_t q = 1; q < p; ++q) acc += parts[(int64_t)q * n + e];
    if (b2) acc += b2[e % d];
    Z[e] = acc;
  }
  return 0;
}

/*
 * The unsharded MLP, fp64, written directly from its definition (it does not
 * call the shard functions): H = X W1 (+ b1), Y = act(H) (or SiLU(X Wg) *
 * (X Wu)), Z = Y W2 (+ b2).  X [T,d], W1 and Wu [d,k], W2 [k,d], Z [T,d].
 */
int oracle_mlp_unsharded_f64(int64_t T, int64_t d, int64_t k, const double *X,
                             const double *W1, const double *Wu, const double *b1,
                             int act, const double *W2, const double *b2, double *Z) {
  if (act == OR_ACT_SWIGLU && Wu == NULL) return -1;
#pragma omp parallel
  {
    double *h = (double *)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
    double *u = (double *)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      for (int64_t j = 0; j < k; ++j) h[j] = 0.0;
      for (int64_t j = 0; j < k; ++j) u[j] = 0.0;
      for (int64_t c = 0; c < d; ++c) {
        const double xv = X[t * d + c];
        for (int64_t j = 0; j < k; ++j) h[j] += xv * W1[c * k + j];
        if (act == OR_ACT_SWIGLU)
          for (int64_t j = 0; j < k; ++j) u[j] += xv * Wu[c * k + j];
      }
      for (int64_t j = 0; j < k; ++j) {
        if (act == OR_ACT_SWIGLU)
          h[j] = act_scalar_f64(OR_ACT_SWIGLU, h[j]) * u[j];
        else
          h[j] = act_scalar_f64(act, b1 ? h[j] + b1[j] : h[j]);
      }
      double *z = Z + t * d;
      for (int64_t n = 0; n < d; ++n) z[n] = 0.0;
      for (int64_t j = 0; j < k; ++j) {
        const double yv = h[j];
        for (int64_t n = 0; n < d; ++n) z[n] += yv * W2[j * d + n];
      }
      if (b2)
        for (int64_t n = 0; n < d; ++n) z[n] += b2[n];
    }
    free(h);
    free(u);
  }
  return 0;
}

/* ---- fp32 instances: the Day 41 post prints its check in fp32 ---------- */

/* Full (unsharded) fp32 linear: Y [T,k] = act(X W + b). */
int oracle_linear_f32(int64_t T, int64_t d, int64_t k, const float *X, const float *W,
                      const float *b, int act, float *Y) {
  if (act == OR_ACT_SWIGLU) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    float *h = Y + t * k;
    for (int64_t j = 0; j < k; ++j) h[j] = 0.0f;
    for (int64_t c = 0; c < d; ++c) {
      const float xv = X[t * d + c];
      for (int64_t j = 0; j < k; ++j) h[j] += xv * W[c * k + j];
    }
    for (int64_t j = 0; j < k; ++j) h[j] = act_scalar_f32(act, b ? h[j] + b[j] : h[j]);
  }
  return 0;
}

/* fp32 column-parallel step of shard i of p (same contract as the fp64 one). */
int oracle_col_shard_f32(int64_t T, int64_t d, int64_t k, int32_t i, int32_t p,
                         const float *X, const float *W1, const float *Wu,
                         const float *b1, int act, float *Y) {
  if (!shard_ok(k, i, p)) return -1;
  if (act == OR_ACT_SWIGLU && Wu == NULL) return -1;
  const int64_t s = k / p, c0 = (int64_t)i * s;
#pragma omp parallel
  {
    float *u = (float *)malloc(sizeof(float) * (size_t)(s > 0 ? s : 1));
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      float *h = Y + t * s;
      for (int64_t j = 0; j < s; ++j) h[j] = 0.0f;
      for (int64_t j = 0; j < s; ++j) u[j] = 0.0f;
      for (int64_t c = 0; c < d; ++c) {
        const float xv = X[t * d + c];
        const float *w = W1 + c * k + c0;
        for (int64_t j = 0; j < s; ++j) h[j] += xv * w[j];
        if (act == OR_ACT_SWIGLU) {
          const float *wu = Wu + c * k + c0;
          for (int64_t j = 0; j < s; ++j) u[j] += xv * wu[j];
        }
      }
      if (act == OR_ACT_SWIGLU) {
        for (int64_t j = 0; j < s; ++j) h[j] = act_scalar_f32(OR_ACT_SWIGLU, h[j]) * u[j];
      } else {
        for (int64_t j = 0; j < s; ++j)
          h[j] = act_scalar_f32(act, b1 ? h[j] + b1[c0 + j] : h[j]);
      }
    }
    free(u);
  }
  return 0;
}

/* fp32 reduction of p partials, shard 0 first, then + b2 (if given). */
int oracle_partial_sum_f32(int64_t T, int64_t d, int32_t p, const float *parts,
                           const float *b2, float *Z) {
  if (p < 1) return -1;
  const int64_t n = T * d;
#pragma omp parallel for schedule(static)
  for (int64_t e = 0; e < n; ++e) {
    float acc = parts[e];
    for (int32_t q = 1; q < p; ++q) acc += parts[(int64_t)q * n + e];
    if (b2) acc += b2[e % d];
    Z[e] = acc;
  }
  return 0;
}

/* ---- attention projections ---------------------------------------------- */

/*
 * Column-parallel QKV projection of shard i of p, fp64.
 *
 * Multi-head attention is split across GPUs by heads: each GPU owns a
 * disjoint, contiguous group of heads and computes the query, key and value
 * projections of those heads alone from the replicated input X ("Transformer
 * math: tensor parallel", section "Attention: parallel across heads";
 * "Tensor Parallelism Explained", section 2.A; "Building GPT from Scratch,
 * Part 9", section "Splitting the Attention Layer").  With grouped key/value
 * heads the key and value heads are split the same way, Hkv/p per GPU
 * ("What is Tensor Parallelism?", section "Worked example: Llama 3.1 70B on 8
 * GPUs").  Both head counts must be divisible by p.
 *
 *   X    [T,d]
 *   W    [d, (Hq + 2 Hkv) dh], the packed projection: query heads in columns
 *        [0, Hq dh), key heads in [Hq dh, (Hq + Hkv) dh), value heads after
 *        that; head h of a part owns the dh columns starting at h dh within it.
 *   b    [(Hq + 2 Hkv) dh] laid out the same way, or NULL.
 *   QKV  [T, (Hq + 2 Hkv) dh / p] receives, per token, the shard's query heads,
 *        then its key heads, then its value heads (in that order, as the
 *        per-GPU projection is split into q, k and v in the Part 9 module),
 *        each head's dh columns in order.
 */
int oracle_qkv_shard_f64(int64_t T, int64_t d, int32_t Hq, int32_t Hkv, int64_t dh, int32_t i,
                         int32_t p, const double *X, const double *W, const double *b,
                         double *QKV) {
  if (p < 1 || i < 0 || i >= p || Hq < 1 || Hkv < 1 || dh < 1) return -1;
  if (Hq % p != 0 || Hkv % p != 0) return -1;
  const int64_t ncol = ((int64_t)Hq + 2 * (int64_t)Hkv) * dh, nout = ncol / p;
  /* The weight column behind each output column, listed part by part, head
     by head. */
  int64_t *src = (int64_t *)malloc(sizeof(int64_t) * (size_t)nout);
  if (!src) return -1;
  int64_t o = 0;
  for (int part = 0; part < 3; ++part) {
    const int64_t heads = part == 0 ? Hq : Hkv;
    const int64_t part_start = part == 0 ? 0 : (part == 1 ? (int64_t)Hq * dh : ((int64_t)Hq + Hkv) * dh);
    const int64_t per_gpu = heads / p;
    for (int64_t h = (int64_t)i * per_gpu; h < ((int64_t)i + 1) * per_gpu; ++h)
      for (int64_t j = 0; j < dh; ++j) src[o++] = part_start + h * dh + j;
  }
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t n = 0; n < nout; ++n) {
      double acc = 0.0;
      for (int64_t c = 0; c < d; ++c) acc += X[t * d + c] * W[c * ncol + src[n]];
      QKV[t * nout + n] = b ? acc + b[src[n]] : acc;
    }
  }
  free(src);
  return 0;
}

/* ---- the backward pass of one MLP shard ---------------------------------- */

/*
 * Derivative of the activation at x (kind 4 is SiLU here), from the
 * definitions above:
 *   GeLU, tanh form: with u = sqrt(2/pi) (x + 0.044715 x^3) and t = tanh(u),
 *                    0.5 (1 + t) + 0.5 x (1 - t^2) sqrt(2/pi) (1 + 3 * 0.044715 x^2)
 *   GeLU, erf form:  Phi(x) + x phi(x) = 0.5 (1 + erf(x / sqrt 2)) + x exp(-x^2 / 2) / sqrt(2 pi)
 *   SiLU:            s (1 + x (1 - s)), s = 1 / (1 + exp(-x))
 *   ReLU:            1 for x > 0, else 0 (0 at x = 0)
 */
static double dact_scalar_f64(int kind, double x) {
  switch (kind) {
    case OR_ACT_NONE:
      return 1.0;
    case OR_ACT_RELU:
      return x > 0.0 ? 1.0 : 0.0;
    case OR_ACT_GELU_TANH: {
      const double c = sqrt(2.0 / M_PI);
      const double t = tanh(c * (x + 0.044715 * x * x * x));
      return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * c * (1.0 + 3.0 * 0.044715 * x * x);
    }
    case OR_ACT_GELU_ERF:
      return 0.5 * (1.0 + erf(x / sqrt(2.0))) + x * exp(-0.5 * x * x) / sqrt(2.0 * M_PI);
    case OR_ACT_SWIGLU: {
      const double s = 1.0 / (1.0 + exp(-x));
      return s * (1.0 + x * (1.0 - s));
    }
  }
  return NAN;
}

/* y[n] = act'(x[n]) (kind 4 is SiLU'). */
void oracle_dactivation_f64(int kind, int64_t n, const double *x, double *y) {
  for (int64_t e = 0; e < n; ++e) y[e] = dact_scalar_f64(kind, x[e]);
}

/*
 * Backward pass of shard i of p, fp64, given the gradient dZ [T,d] of the
 * loss with respect to the block output Z = sum_i Z_i.
 *
 * The reduction after the row-parallel step passes the same dZ to every
 * shard (its backward is the identity), and the row-parallel step's input
 * gradient is local: dY_i = dZ B_i^T.  The activation is element-wise, so
 * dH_i = dY_i * act'(H_i) is local too.  The column-parallel step's input
 * gradient is one term of a sum over the shards, dX = sum_i dH_i A_i^T, which
 * is what the all-reduce before the block adds up ("Transformer math: tensor
 * parallel", sections "Column-parallel: split the weight by output columns",
 * "Row-parallel: split the weight by input rows" and "The f and g conjugate
 * operators").  The weight gradients follow from Y_i = act(X A_i + b1_i) and
 * Z_i = Y_i B_i: dA_i = X^T dH_i, db1_i = column sums of dH_i, dB_i = Y_i^T dZ.
 * For the gated variant Y_i = SiLU(G_i) * U_i with G_i = X Wg_i, U_i = X Wu_i:
 * dG_i = dY_i * U_i * SiLU'(G_i), dU_i = dY_i * SiLU(G_i),
 * dX_i = dG_i Wg_i^T + dU_i Wu_i^T, dWg_i = X^T dG_i, dWu_i = X^T dU_i.
 *
 * The pre-activations are computed here from X and the weights (nothing is
 * taken from a forward run).  Inputs are the full matrices (as the forward
 * functions take them); outputs are compact:
 *   dH  [T,s] (gated: [T,2s], dG_i in columns [0,s), dU_i in [s,2s))
 *   dXp [T,d]   this shard's term of dX
 *   dW1 [d,s]   (gated: dWg_i)       dWu [d,s] (gated only, else unused)
 *   db1 [s] or NULL (not with the gated variant)
 *   dW2 [s,d]
 * Every sum runs with its index ascending (dXp: over the gate columns, then
 * over the up columns).
 */
int oracle_mlp_shard_backward_f64(int64_t T, int64_t d, int64_t k, int32_t i, int32_t p,
                                  const double *X, const double *W1, const double *Wu,
                                  const double *b1, int act, const double *W2, const double *dZ,
                                  double *dH, double *dXp, double *dW1, double *dWu, double *db1,
                                  double *dW2) {
  if (!shard_ok(k, i, p)) return -1;
  const int gated = act == OR_ACT_SWIGLU;
  if (gated && (Wu == NULL || dWu == NULL || db1 != NULL)) return -1;
  const int64_t s = k / p, c0 = (int64_t)i * s, hw = gated ? 2 * s : s;
  const size_t ts = (size_t)(T > 0 ? T : 1) * (size_t)(s > 0 ? s : 1);
  double *H = (double *)malloc(sizeof(double) * ts);  /* pre-activation (gate for SwiGLU) */
  double *U = (double *)malloc(sizeof(double) * ts);  /* up projection (SwiGLU)           */
  double *Y = (double *)malloc(sizeof(double) * ts);  /* activation output               */
  if (!H || !U || !Y) {
    free(H);
    free(U);
    free(Y);
    return -1;
  }
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t j = 0; j < s; ++j) {
      double h = 0.0, u = 0.0, dy = 0.0;
      for (int64_t c = 0; c < d; ++c) h += X[t * d + c] * W1[c * k + c0 + j];
      if (gated)
        for (int64_t c = 0; c < d; ++c) u += X[t * d + c] * Wu[c * k + c0 + j];
      else if (b1)
        h += b1[c0 + j];
      for (int64_t n = 0; n < d; ++n) dy += dZ[t * d + n] * W2[(c0 + j) * d + n];
      H[t * s + j] = h;
      U[t * s + j] = u;
      if (gated) {
        const double sg = act_scalar_f64(OR_ACT_SWIGLU, h);
        Y[t * s + j] = sg * u;
        dH[t * hw + j] = dy * u * dact_scalar_f64(OR_ACT_SWIGLU, h);
        dH[t * hw + s + j] = dy * sg;
      } else {
        Y[t * s + j] = act_scalar_f64(act, h);
        dH[t * hw + j] = dy * dact_scalar_f64(act, h);
      }
    }
  }
  /* dX_i = dH_i W1_i^T (+ dU_i Wu_i^T) */
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t)
    for (int64_t c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int64_t j = 0; j < s; ++j) acc += dH[t * hw + j] * W1[c * k + c0 + j];
      if (gated)
        for (int64_t j = 0; j < s; ++j) acc += dH[t * hw + s + j] * Wu[c * k + c0 + j];
      dXp[t * d + c] = acc;
    }
  /* dW1_i = X^T dH_i, dWu_i = X^T dU_i */
#pragma omp parallel for schedule(static)
  for (int64_t c = 0; c < d; ++c)
    for (int64_t j = 0; j < s; ++j) {
      double a = 0.0, b = 0.0;
      for (int64_t t = 0; t < T; ++t) {
        a += X[t * d + c] * dH[t * hw + j];
        if (gated) b += X[t * d + c] * dH[t * hw + s + j];
      }
      dW1[c * s + j] = a;
      if (gated) dWu[c * s + j] = b;
    }
  if (db1)
    for (int64_t j = 0; j < s; ++j) {
      double a = 0.0;
      for (int64_t t = 0; t < T; ++t) a += dH[t * hw + j];
      db1[j] = a;
    }
  /* dW2_i = Y_i^T dZ */
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < s; ++j)
    for (int64_t n = 0; n < d; ++n) {
      double a = 0.0;
      for (int64_t t = 0; t < T; ++t) a += Y[t * s + j] * dZ[t * d + n];
      dW2[j * d + n] = a;
    }
  free(H);
  free(U);
  free(Y);
  return 0;
}

/* ---- the attention core between the projections -------------------------- */

/*
 * Scaled dot-product attention of one head shard, fp64: for every sequence,
 * query head h and query token t,
 *   s_j  = (Q[t, h] . K[j, c]) / sqrt(dh)     for the keys j the query sees
 *   O[t, h] = sum_j softmax(s)_j V[j, c]
 * with c = h / (Hq / Hkv) the key/value head that query head h reads
 * (grouped heads; c = h when Hq = Hkv).  Heads never mix, so a GPU that owns
 * a group of heads computes their attention alone ("Transformer math: tensor
 * parallel", section "Attention: parallel across heads", which writes the
 * per-head softmax(Q K^T / sqrt(d_k)) V).  With causal != 0 token t of a
 * sequence sees the keys 0..t of that sequence (the causal self-attention of
 * "Building GPT from Scratch, Part 9"); otherwise every key of its sequence.
 * The T = nseq * S tokens form nseq sequences of S consecutive tokens.
 *   Q [T, Hq dh] (head h in columns [h dh, (h+1) dh)), K and V [T, Hkv dh],
 *   O [T, Hq dh], all dense.
 * The softmax subtracts the largest score before exponentiating.
 */
int oracle_attention_f64(int64_t nseq, int64_t S, int32_t Hq, int32_t Hkv, int64_t dh, int causal,
                         const double *Q, const double *K, const double *V, double *O) {
  if (nseq < 0 || S < 0 || Hq < 1 || Hkv < 1 || dh < 1 || Hq % Hkv != 0) return -1;
  const int64_t group = Hq / Hkv, qw = (int64_t)Hq * dh, kw = (int64_t)Hkv * dh;
  const double scale = 1.0 / sqrt((double)dh);
#pragma omp parallel
  {
    double *sc = (double *)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
#pragma omp for collapse(2) schedule(static)
    for (int64_t b = 0; b < nseq; ++b)
      for (int64_t h = 0; h < Hq; ++h) {
        const int64_t c = h / group;
        for (int64_t t = 0; t < S; ++t) {
          const int64_t tq = b * S + t;
          const int64_t nk = causal ? t + 1 : S;
          double mx = -INFINITY;
          for (int64_t j = 0; j < nk; ++j) {
            const int64_t tk = b * S + j;
            double dot = 0.0;
            for (int64_t e = 0; e < dh; ++e) dot += Q[tq * qw + h * dh + e] * K[tk * kw + c * dh + e];
            sc[j] = dot * scale;
            if (sc[j] > mx) mx = sc[j];
          }
          double den = 0.0;
          for (int64_t j = 0; j < nk; ++j) {
            sc[j] = exp(sc[j] - mx);
            den += sc[j];
          }
          for (int64_t e = 0; e < dh; ++e) {
            double acc = 0.0;
            for (int64_t j = 0; j < nk; ++j) acc += sc[j] * V[(b * S + j) * kw + c * dh + e];
            O[tq * qw + h * dh + e] = acc / den;
          }
        }
      }
    free(sc);
  }
  return 0;
}

/* ---- one transformer block ------------------------------------------------ */

/*
 * LayerNorm of each row of X [T,d], fp64: with the row's mean
 *   mu = (1/d) sum_c x_c   and its (biased) variance   var = (1/d) sum_c (x_c - mu)^2,
 *   Y[t,c] = (x_c - mu) / sqrt(var + eps) * gamma[c] + beta[c].
 * The pages name the normalisation only ("Building GPT from Scratch, Part 9",
 * section "Communication Pattern per Transformer Block": a LayerNorm before
 * attention and one before the FFN, replicated on every GPU); this is the
 * standard definition (Ba, Kiros and Hinton, 2016) with a learned scale and
 * shift.
 */
int oracle_layernorm_f64(int64_t T, int64_t d, const double *X, const double *gamma,
                         const double *beta, double eps, double *Y) {
  if (T < 0 || d < 1) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    const double *x = X + t * d;
    double sum = 0.0;
    for (int64_t c = 0; c < d; ++c) sum += x[c];
    const double mu = sum / (double)d;
    double sq = 0.0;
    for (int64_t c = 0; c < d; ++c) sq += (x[c] - mu) * (x[c] - mu);
    const double var = sq / (double)d;
    const double rstd = 1.0 / sqrt(var + eps);
    for (int64_t c = 0; c < d; ++c) Y[t * d + c] = (x[c] - mu) * rstd * gamma[c] + beta[c];
  }
  return 0;
}

/*
 * Rounding to bf16 for the block's mirror mode (a diagnostic, off by
 * default): the value is rounded to fp32 (the precision the GPU's
 * accumulators hold), then to the nearest bf16 with ties to even -- add half
 * of the dropped 16 bits' range, less one, plus the lowest kept bit, and drop
 * those bits.  Non-finite values pass through.
 */
static double bf16_round(double x) {
  float f = (float)x;
  if (!isfinite(f)) return f;
  uint32_t b;
  memcpy(&b, &f, 4);
  b += 0x7fffu + ((b >> 16) & 1u);
  b &= 0xffff0000u;
  memcpy(&f, &b, 4);
  return (double)f;
}

void oracle_round_bf16_f64(int64_t n, const double *x, double *y) {
  for (int64_t e = 0; e < n; ++e) y[e] = bf16_round(x[e]);
}

/*
 * One pre-LayerNorm transformer block, unsharded, fp64, in the order of
 * "Building GPT from Scratch, Part 9", section "Communication Pattern per
 * Transformer Block" (LayerNorm, attention, residual add, LayerNorm, FFN,
 * residual add):
 *   A   = LN1(X)
 *   QKV = A Wqkv + bqkv          Wqkv [d, (Hq + 2 Hkv) dh]: all query heads,
 *                                then all key heads, then all value heads
 *   O   = attention(Q, K, V)     as oracle_attention_f64 (nseq sequences of S)
 *   X1  = X + (O WO + bO)        WO [Hq dh, d]
 *   B   = LN2(X1)
 *   Out = X1 + MLP(B)            MLP as oracle_mlp_unsharded_f64, with b2
 * X [T,d] with T = nseq S.  The attention half is computed for every token
 * (keys come from all of them); the FFN half only for the nrows tokens listed
 * in rows (rows == NULL: all T, in order).  Out [nrows, d].  bqkv, bO, b1 and
 * b2 may be NULL (no bias); Wu only for act = OR_ACT_SWIGLU.
 * mirror != 0 (diagnostic only) rounds to bf16 the activations a bf16
 * implementation stores: A, QKV, O, B and the FFN hidden activation; the
 * residual stream and everything else stay fp64.
 */
int oracle_block_f64(int64_t nseq, int64_t S, int64_t d, int32_t Hq, int32_t Hkv, int64_t dh,
                     int64_t k, int causal, int act, double eps, const double *X,
                     const double *ln1_g, const double *ln1_b, const double *Wqkv,
                     const double *bqkv, const double *WO, const double *bO,
                     const double *ln2_g, const double *ln2_b, const double *W1,
                     const double *Wu, const double *b1, const double *W2, const double *b2,
                     int mirror, int64_t nrows, const int64_t *rows, double *Out) {
  if (nseq < 0 || S < 0 || d < 1 || Hq < 1 || Hkv < 1 || dh < 1 || k < 1 || Hq % Hkv) return -1;
  if (act == OR_ACT_SWIGLU && Wu == NULL) return -1;
  const int64_t T = nseq * S, ncol = ((int64_t)Hq + 2 * (int64_t)Hkv) * dh;
  const int64_t qw = (int64_t)Hq * dh, kw = (int64_t)Hkv * dh;
  if (rows == NULL) nrows = T;
  for (int64_t r = 0; r < nrows; ++r)
    if (rows && (rows[r] < 0 || rows[r] >= T)) return -1;
  double *A = (double *)malloc(sizeof(double) * (size_t)(T * d + 1));
  double *QKV = (double *)malloc(sizeof(double) * (size_t)(T * ncol + 1));
  double *Q = (double *)malloc(sizeof(double) * (size_t)(T * qw + 1));
  double *K = (double *)malloc(sizeof(double) * (size_t)(T * kw + 1));
  double *V = (double *)malloc(sizeof(double) * (size_t)(T * kw + 1));
  double *O = (double *)malloc(sizeof(double) * (size_t)(T * qw + 1));
  double *X1 = (double *)malloc(sizeof(double) * (size_t)(nrows * d + 1));
  double *B = (double *)malloc(sizeof(double) * (size_t)(nrows * d + 1));
  double *Z = (double *)malloc(sizeof(double) * (size_t)(nrows * d + 1));
  int rc = -1;
  if (!A || !QKV || !Q || !K || !V || !O || !X1 || !B || !Z) goto out;
  if (oracle_layernorm_f64(T, d, X, ln1_g, ln1_b, eps, A)) goto out;
  if (mirror)
    for (int64_t e = 0; e < T * d; ++e) A[e] = bf16_round(A[e]);
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    double *q = QKV + t * ncol;
    for (int64_t n = 0; n < ncol; ++n) q[n] = 0.0;
    for (int64_t c = 0; c < d; ++c) {
      const double av = A[t * d + c];
      const double *w = Wqkv + c * ncol;
      for (int64_t n = 0; n < ncol; ++n) q[n] += av * w[n];
    }
    if (bqkv)
      for (int64_t n = 0; n < ncol; ++n) q[n] += bqkv[n];
    if (mirror)
      for (int64_t n = 0; n < ncol; ++n) q[n] = bf16_round(q[n]);
    memcpy(Q + t * qw, q, sizeof(double) * (size_t)qw);
    memcpy(K + t * kw, q + qw, sizeof(double) * (size_t)kw);
    memcpy(V + t * kw, q + qw + kw, sizeof(double) * (size_t)kw);
  }
  if (oracle_attention_f64(nseq, S, Hq, Hkv, dh, causal, Q, K, V, O)) goto out;
  if (mirror)
    for (int64_t e = 0; e < T * qw; ++e) O[e] = bf16_round(O[e]);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t t = rows ? rows[r] : r;
    double *x1 = X1 + r * d;
    for (int64_t n = 0; n < d; ++n) x1[n] = 0.0;
    for (int64_t j = 0; j < qw; ++j) {
      const double ov = O[t * qw + j];
      const double *w = WO + j * d;
      for (int64_t n = 0; n < d; ++n) x1[n] += ov * w[n];
    }
    for (int64_t n = 0; n < d; ++n) x1[n] = X[t * d + n] + (bO ? x1[n] + bO[n] : x1[n]);
  }
  if (oracle_layernorm_f64(nrows, d, X1, ln2_g, ln2_b, eps, B)) goto out;
  if (mirror)
    for (int64_t e = 0; e < nrows * d; ++e) B[e] = bf16_round(B[e]);
  /* The FFN of the listed rows: Y = act(B W1 + b1) (or SiLU(B Wg) * (B Wu)),
     Z = Y W2 + b2, each dot product over its index ascending. */
#pragma omp parallel
  {
    double *hid = (double *)malloc(sizeof(double) * (size_t)k);
    double *up = (double *)malloc(sizeof(double) * (size_t)k);
#pragma omp for schedule(static)
    for (int64_t r = 0; r < nrows; ++r) {
      for (int64_t j = 0; j < k; ++j) hid[j] = up[j] = 0.0;
      for (int64_t c = 0; c < d; ++c) {
        const double bv = B[r * d + c];
        for (int64_t j = 0; j < k; ++j) hid[j] += bv * W1[c * k + j];
        if (act == OR_ACT_SWIGLU)
          for (int64_t j = 0; j < k; ++j) up[j] += bv * Wu[c * k + j];
      }
      for (int64_t j = 0; j < k; ++j) {
        const double y = act == OR_ACT_SWIGLU ? act_scalar_f64(OR_ACT_SWIGLU, hid[j]) * up[j]
                                              : act_scalar_f64(act, b1 ? hid[j] + b1[j] : hid[j]);
        hid[j] = mirror ? bf16_round(y) : y;
      }
      double *z = Z + r * d;
      for (int64_t n = 0; n < d; ++n) z[n] = 0.0;
      for (int64_t j = 0; j < k; ++j) {
        const double *w = W2 + j * d;
        for (int64_t n = 0; n < d; ++n) z[n] += hid[j] * w[n];
      }
      if (b2)
        for (int64_t n = 0; n < d; ++n) z[n] += b2[n];
    }
    free(hid);
    free(up);
  }
  for (int64_t e = 0; e < nrows * d; ++e) Out[e] = X1[e] + Z[e];
  rc = 0;
out:
  free(A);
  free(QKV);
  free(Q);
  free(K);
  free(V);
  free(O);
  free(X1);
  free(B);
  free(Z);
  return rc;
}
