// Host side of libtpmlp: argument checks, shard bookkeeping, path choice and
// launches on the caller's stream.  Every check happens before any launch, so
// an error status means nothing was enqueued and no output was touched.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/tpmlp.h"
#include "../../include/tpmlp_calib.h"
#include "kernels.h"

using namespace tpmlp;

namespace {

thread_local std::string g_msg;

tp_status fail(tp_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_msg = buf;
  return s;
}

tp_status ok() {
  g_msg.clear();
  return TP_OK;
}

// Few-token path threshold: at or below this many tokens the shard is a
// weight-streaming problem (HBM-bound), above it a tiled MFMA problem.
constexpr int64_t kDecodeMaxT = 64;
// Column blocks of 128 the few-token path's workspace counters can track.
constexpr int64_t kDecodeMaxCols = 65536 * 128;

size_t elem_size(tp_dtype dt) { return dt == TP_BF16 ? 2 : 4; }
int64_t elem_align(tp_dtype dt) { return dt == TP_BF16 ? 8 : 4; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

tp_status check_dtype_act(tp_dtype dt, int act) {
  if (dt != TP_F32 && dt != TP_BF16) return fail(TP_ERR_BAD_DTYPE, "unknown dtype %d", (int)dt);
  if (act < TP_ACT_NONE || act > TP_ACT_SWIGLU)
    return fail(TP_ERR_BAD_ACT, "unknown activation %d", act);
  return TP_OK;
}

// Shape and shard rule shared by every shard entry point.
tp_status check_shard(int64_t T, int64_t d, int64_t k, int32_t i, int32_t p) {
  if (T < 0) return fail(TP_ERR_BAD_SHAPE, "T = %lld < 0", (long long)T);
  if (d < 1) return fail(TP_ERR_BAD_SHAPE, "d = %lld < 1", (long long)d);
  if (k < 1) return fail(TP_ERR_BAD_SHAPE, "k = %lld < 1", (long long)k);
  if (p < 1 || p > TP_MAX_SHARDS)
    return fail(TP_ERR_BAD_SHARD, "p = %d outside [1, %d]", p, TP_MAX_SHARDS);
  if (i < 0 || i >= p) return fail(TP_ERR_BAD_SHARD, "shard index i = %d outside [0, %d)", i, p);
  if (k % p != 0)
    return fail(TP_ERR_NOT_DIVISIBLE, "k = %lld is not divisible by p = %d", (long long)k, p);
  return TP_OK;
}

tp_status check_ld(const char *name, int64_t ld, int64_t width, tp_dtype dt) {
  if (ld < width)
    return fail(TP_ERR_BAD_SHAPE, "%s = %lld is below the row width %lld", name, (long long)ld,
                (long long)width);
  if (ld % elem_align(dt) != 0)
    return fail(TP_ERR_MISALIGNED, "%s = %lld is not a multiple of %lld elements", name,
                (long long)ld, (long long)elem_align(dt));
  return TP_OK;
}

tp_status check_ptr(const char *name, const void *ptr) {
  if (!ptr) return fail(TP_ERR_NULL_POINTER, "%s is NULL", name);
  if (!aligned16(ptr)) return fail(TP_ERR_MISALIGNED, "%s is not 16-byte aligned", name);
  return TP_OK;
}

#define TRY(expr)                   \
  do {                              \
    const tp_status st_ = (expr);   \
    if (st_ != TP_OK) return st_;   \
  } while (0)

struct ColCall {
  tp_dtype dt;
  int act;
  int64_t T, d, k;
  int32_t i, p;
  const void *X, *W1, *Wu, *b1;
  int64_t ldx, ldw1, ldwu, ldy;
  void *Y;
};

tp_status validate_col(const ColCall &c) {
  TRY(check_dtype_act(c.dt, c.act));
  TRY(check_shard(c.T, c.d, c.k, c.i, c.p));
  const int64_t s = c.k / c.p;
  if (c.d % elem_align(c.dt) || s % elem_align(c.dt))
    return fail(TP_ERR_MISALIGNED, "d = %lld and k/p = %lld must be multiples of %lld",
                (long long)c.d, (long long)s, (long long)elem_align(c.dt));
  if (c.T > 0) {  // with no tokens X and Y are never touched and may be NULL
    TRY(check_ptr("X", c.X));
    TRY(check_ptr("Y", c.Y));
  }
  TRY(check_ptr("W1", c.W1));
  TRY(check_ld("ldx", c.ldx, c.d, c.dt));
  TRY(check_ld("ldw1", c.ldw1, c.k, c.dt));
  TRY(check_ld("ldy", c.ldy, s, c.dt));
  if (c.act == TP_ACT_SWIGLU) {
    TRY(check_ptr("Wu", c.Wu));
    TRY(check_ld("ldwu", c.ldwu, c.k, c.dt));
    if (c.b1) return fail(TP_ERR_BAD_ACT, "a column bias is not supported with SWIGLU");
  } else if (c.b1) {
    TRY(check_ptr("b1", c.b1));
  }
  return TP_OK;
}

struct RowCall {
  tp_dtype dt;
  int64_t T, d, k;
  int32_t i, p;
  const void *Y, *W2;
  int64_t ldy, ldw2, ldz;
  float *Z;
};

tp_status validate_row(const RowCall &r) {
  TRY(check_dtype_act(r.dt, TP_ACT_NONE));
  TRY(check_shard(r.T, r.d, r.k, r.i, r.p));
  const int64_t s = r.k / r.p;
  if (r.d % elem_align(r.dt) || s % elem_align(r.dt))
    return fail(TP_ERR_MISALIGNED, "d = %lld and k/p = %lld must be multiples of %lld",
                (long long)r.d, (long long)s, (long long)elem_align(r.dt));
  if (r.T > 0) {  // with no tokens Y and Z are never touched and may be NULL
    TRY(check_ptr("Y", r.Y));
    TRY(check_ptr("Z", r.Z));
  }
  TRY(check_ptr("W2", r.W2));
  TRY(check_ld("ldy", r.ldy, s, r.dt));
  TRY(check_ld("ldw2", r.ldw2, r.d, r.dt));
  TRY(check_ld("ldz", r.ldz, r.d, TP_F32));
  return TP_OK;
}

// GEMM descriptors of one shard (or of all p shards, grouped).  The column
// block of W1/Wu/b1 of shard i starts at column i*s, the row block of W2 at
// row i*s (Day 41 post, "Simulating column parallel linear" and "Simulating
// row parallel linear").
GemmArgs col_gemm(const ColCall &c, int groups, int64_t ystride) {
  const int64_t s = c.k / c.p, c0 = (int64_t)c.i * s;
  const size_t es = elem_size(c.dt);
  GemmArgs a{};
  a.A = c.X;
  a.lda = c.ldx;
  a.B = (const char *)c.W1 + c0 * es;
  a.ldb = c.ldw1;
  a.B2 = c.Wu ? (const void *)((const char *)c.Wu + c0 * es) : nullptr;
  a.ldb2 = c.ldwu;
  a.bias = c.b1 ? (const void *)((const char *)c.b1 + c0 * es) : nullptr;
  a.C = c.Y;
  a.ldc = c.ldy;
  a.M = c.T;
  a.N = s;
  a.K = c.d;
  a.epi = c.act == TP_ACT_SWIGLU ? EPI_SWIGLU : EPI_ACT;
  a.act = c.act;
  a.groups = groups;
  a.sA = 0;
  a.sB = s;
  a.sB2 = s;
  a.sBias = s;
  a.sC = ystride;
  return a;
}

GemmArgs row_gemm(const RowCall &r, int groups, int64_t ystride, int64_t zstride) {
  const int64_t s = r.k / r.p, c0 = (int64_t)r.i * s;
  GemmArgs a{};
  a.A = r.Y;
  a.lda = r.ldy;
  a.B = (const char *)r.W2 + c0 * r.ldw2 * elem_size(r.dt);
  a.ldb = r.ldw2;
  a.C = r.Z;
  a.ldc = r.ldz;
  a.M = r.T;
  a.N = r.d;
  a.K = s;
  a.epi = EPI_F32;
  a.act = TP_ACT_NONE;
  a.groups = groups;
  a.sA = ystride;
  a.sB = s * r.ldw2;
  a.sC = zstride;
  return a;
}

// Workspace of one bf16 GEMM: the few-token path's split-K partials, or the
// tiled path's when it splits K (problems with few tiles).
size_t gemm_ws_bytes(tp_dtype dt, const GemmArgs &a) {
  if (dt != TP_BF16 || a.M <= 0) return 0;
  return a.M <= kDecodeMaxT ? decode_workspace_bytes(a) : tiled_workspace_bytes(a);
}

// The bf16 kernels address memory with 32-bit buffer offsets from a tile's or
// stage's base; shapes beyond that range are rejected here, before any launch.
tp_status check_gemm(tp_dtype dt, const GemmArgs &a) {
  if (dt != TP_BF16 || a.M <= 0) return TP_OK;
  const bool fits =
      a.M <= kDecodeMaxT ? gemm_bf16_decode_supported(a) : gemm_bf16_tiled_supported(a);
  if (!fits)
    return fail(TP_ERR_BAD_SHAPE,
                "shape beyond the bf16 kernels' offset range: leading dimensions must be below "
                "2^21 (X, more than 64 tokens) or 2^23 elements, and at most %lld output columns "
                "with 64 or fewer tokens",
                (long long)kDecodeMaxCols);
  return TP_OK;
}

tp_status run_gemm(tp_dtype dt, const GemmArgs &a, void *ws, hipStream_t st) {
  hipError_t e;
  if (dt == TP_F32)
    e = launch_gemm_f32(a, st);
  else if (a.M <= kDecodeMaxT)
    e = launch_gemm_bf16_decode(a, ws, st);
  else
    e = launch_gemm_bf16_tiled(a, ws, st);
  if (e != hipSuccess) return fail(TP_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return TP_OK;
}

// The workspace a GEMM needs given the caller's buffer.  The tiled path
// (more than 64 tokens) splits K only when the buffer holds the partials; with
// no buffer, or a smaller one, it runs unsplit (a.splitk = 1) and needs none.
// The few-token path has no unsplit form: its need stands.
size_t fit_gemm_ws(tp_dtype dt, GemmArgs &a, const void *ws, size_t ws_bytes) {
  const size_t need = gemm_ws_bytes(dt, a);
  if (need > 0 && dt == TP_BF16 && a.M > kDecodeMaxT && (!ws || ws_bytes < need)) {
    a.splitk = 1;
    return gemm_ws_bytes(dt, a);
  }
  return need;
}

tp_status check_ws(size_t need, void *ws, size_t ws_bytes) {
  if (need == 0) return TP_OK;
  if (!ws || ws_bytes < need)
    return fail(TP_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", need,
                ws ? ws_bytes : (size_t)0);
  if (!aligned16(ws)) return fail(TP_ERR_MISALIGNED, "workspace is not 16-byte aligned");
  return TP_OK;
}

ColCall make_col(tp_dtype dt, tp_act act, int64_t T, int64_t d, int64_t k, int32_t i, int32_t p,
                 const void *X, int64_t ldx, const void *W1, int64_t ldw1, const void *Wu,
                 int64_t ldwu, const void *b1, void *Y, int64_t ldy) {
  ColCall c;
  c.dt = dt;
  c.act = (int)act;
  c.T = T;
  c.d = d;
  c.k = k;
  c.i = i;
  c.p = p;
  c.X = X;
  c.W1 = W1;
  c.Wu = (act == TP_ACT_SWIGLU) ? Wu : nullptr;
  c.b1 = b1;
  c.ldx = ldx;
  c.ldw1 = ldw1;
  c.ldwu = ldwu;
  c.ldy = ldy;
  c.Y = Y;
  return c;
}

RowCall make_row(tp_dtype dt, int64_t T, int64_t d, int64_t k, int32_t i, int32_t p,
                 const void *Y, int64_t ldy, const void *W2, int64_t ldw2, float *Z, int64_t ldz) {
  RowCall r;
  r.dt = dt;
  r.T = T;
  r.d = d;
  r.k = k;
  r.i = i;
  r.p = p;
  r.Y = Y;
  r.W2 = W2;
  r.ldy = ldy;
  r.ldw2 = ldw2;
  r.ldz = ldz;
  r.Z = Z;
  return r;
}

size_t max_sz(size_t a, size_t b) { return a > b ? a : b; }

struct QkvCall {
  tp_dtype dt;
  int64_t T, d;
  int32_t Hq, Hkv;
  int64_t dh;
  int32_t i, p;
  const void *X, *W, *b;
  int64_t ldx, ldw, ldo;
  void *QKV;
};

tp_status validate_qkv(const QkvCall &c) {
  TRY(check_dtype_act(c.dt, TP_ACT_NONE));
  if (c.T < 0) return fail(TP_ERR_BAD_SHAPE, "T = %lld < 0", (long long)c.T);
  if (c.d < 1) return fail(TP_ERR_BAD_SHAPE, "d = %lld < 1", (long long)c.d);
  if (c.Hq < 1 || c.Hkv < 1 || c.dh < 1)
    return fail(TP_ERR_BAD_SHAPE, "Hq = %d, Hkv = %d and dh = %lld must be >= 1", c.Hq, c.Hkv,
                (long long)c.dh);
  if (c.p < 1 || c.p > TP_MAX_SHARDS)
    return fail(TP_ERR_BAD_SHARD, "p = %d outside [1, %d]", c.p, TP_MAX_SHARDS);
  if (c.i < 0 || c.i >= c.p)
    return fail(TP_ERR_BAD_SHARD, "shard index i = %d outside [0, %d)", c.i, c.p);
  if (c.Hq % c.p || c.Hkv % c.p)
    return fail(TP_ERR_NOT_DIVISIBLE, "head counts Hq = %d and Hkv = %d must be divisible by p = %d",
                c.Hq, c.Hkv, c.p);
  if (c.d % elem_align(c.dt) || c.dh % elem_align(c.dt))
    return fail(TP_ERR_MISALIGNED, "d = %lld and dh = %lld must be multiples of %lld",
                (long long)c.d, (long long)c.dh, (long long)elem_align(c.dt));
  const int64_t ncol = ((int64_t)c.Hq + 2 * (int64_t)c.Hkv) * c.dh;
  if (c.T > 0) {  // with no tokens X and QKV are never touched and may be NULL
    TRY(check_ptr("X", c.X));
    TRY(check_ptr("QKV", c.QKV));
  }
  TRY(check_ptr("Wqkv", c.W));
  if (c.b) TRY(check_ptr("bqkv", c.b));
  TRY(check_ld("ldx", c.ldx, c.d, c.dt));
  TRY(check_ld("ldw", c.ldw, ncol, c.dt));
  TRY(check_ld("ldo", c.ldo, ncol / c.p, c.dt));
  return TP_OK;
}

// The QKV projection of head shard i is a column-parallel linear whose output
// columns come from three column blocks of the packed weight: the shard's
// query heads, its key heads and its value heads ("Transformer math: tensor
// parallel", section "Attention: parallel across heads").  One GEMM with a
// three-segment column map computes all three.
GemmArgs qkv_gemm(const QkvCall &c) {
  const int64_t qw = (int64_t)c.Hq * c.dh / c.p, kw = (int64_t)c.Hkv * c.dh / c.p;
  GemmArgs a{};
  a.A = c.X;
  a.lda = c.ldx;
  a.B = c.W;
  a.ldb = c.ldw;
  a.bias = c.b;
  a.C = c.QKV;
  a.ldc = c.ldo;
  a.M = c.T;
  a.N = qw + 2 * kw;
  a.K = c.d;
  a.epi = EPI_ACT;
  a.act = TP_ACT_NONE;
  a.groups = 1;
  a.nseg = 3;
  a.seg_start[0] = 0;
  a.seg_start[1] = qw;
  a.seg_start[2] = qw + kw;
  a.seg_src[0] = c.i * qw;
  a.seg_src[1] = (int64_t)c.Hq * c.dh + c.i * kw;
  a.seg_src[2] = ((int64_t)c.Hq + c.Hkv) * c.dh + c.i * kw;
  return a;
}

// The backward pass and the forward that keeps what it needs always run the
// tiled kernels (bf16) or the fp32 kernels, whatever T: they need the
// transposed-operand layouts and epilogues only those have.
tp_status check_tiled(tp_dtype dt, const GemmArgs &a) {
  if (dt != TP_BF16) return TP_OK;
  if (!gemm_bf16_tiled_supported(a))
    return fail(TP_ERR_BAD_SHAPE,
                "shape beyond the bf16 kernels' offset range: leading dimensions must be below "
                "2^21 elements (2^23 for weights), and a transposed weight block below 2^30");
  return TP_OK;
}

tp_status run_tiled(tp_dtype dt, const GemmArgs &a, hipStream_t st) {
  // (the backward's layouts and epilogues never split K: no workspace)
  const hipError_t e =
      dt == TP_F32 ? launch_gemm_f32(a, st) : launch_gemm_bf16_tiled(a, nullptr, st);
  if (e != hipSuccess) return fail(TP_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return TP_OK;
}

struct BwdCall {
  tp_dtype dt;
  int act;
  int64_t T, d, k;
  int32_t i, p;
  const void *X, *W1, *Wu, *W2, *H, *Y, *dZ;
  int64_t ldx, ldw1, ldwu, ldw2, ldh, ldy, lddz;
  void *dH;
  int64_t lddh;
  float *dXp, *dW1, *dWu, *db1, *dW2;
  int64_t lddx, lddw1, lddwu, lddw2;
};

tp_status validate_bwd(const BwdCall &c) {
  TRY(check_dtype_act(c.dt, c.act));
  TRY(check_shard(c.T, c.d, c.k, c.i, c.p));
  const int64_t s = c.k / c.p;
  const bool gated = c.act == TP_ACT_SWIGLU;
  const int64_t hw = gated ? 2 * s : s;
  if (c.d % elem_align(c.dt) || s % elem_align(c.dt))
    return fail(TP_ERR_MISALIGNED, "d = %lld and k/p = %lld must be multiples of %lld",
                (long long)c.d, (long long)s, (long long)elem_align(c.dt));
  if (c.T > 0) {  // token-sized buffers are never touched with no tokens
    TRY(check_ptr("X", c.X));
    TRY(check_ptr("H", c.H));
    TRY(check_ptr("Y", c.Y));
    TRY(check_ptr("dZ", c.dZ));
    TRY(check_ptr("dH", c.dH));
    TRY(check_ptr("dXp", c.dXp));
  }
  TRY(check_ptr("W1", c.W1));
  TRY(check_ptr("W2", c.W2));
  TRY(check_ptr("dW1", c.dW1));
  TRY(check_ptr("dW2", c.dW2));
  TRY(check_ld("ldx", c.ldx, c.d, c.dt));
  TRY(check_ld("ldw1", c.ldw1, c.k, c.dt));
  TRY(check_ld("ldw2", c.ldw2, c.d, c.dt));
  TRY(check_ld("ldh", c.ldh, hw, c.dt));
  TRY(check_ld("ldy", c.ldy, s, c.dt));
  TRY(check_ld("lddz", c.lddz, c.d, c.dt));
  TRY(check_ld("lddh", c.lddh, hw, c.dt));
  TRY(check_ld("lddx", c.lddx, c.d, TP_F32));
  TRY(check_ld("lddw1", c.lddw1, s, TP_F32));
  TRY(check_ld("lddw2", c.lddw2, c.d, TP_F32));
  if (gated) {
    TRY(check_ptr("Wu", c.Wu));
    TRY(check_ptr("dWu", c.dWu));
    TRY(check_ld("ldwu", c.ldwu, c.k, c.dt));
    TRY(check_ld("lddwu", c.lddwu, s, TP_F32));
    if (c.db1) return fail(TP_ERR_BAD_ACT, "a column bias gradient is not defined with SWIGLU");
  } else if (c.db1) {
    TRY(check_ptr("db1", c.db1));
  }
  return TP_OK;
}

// The GEMMs of the backward pass of shard i ("Transformer math: tensor
// parallel", sections "Column-parallel: split the weight by output columns",
// "Row-parallel: split the weight by input rows" and "The f and g conjugate
// operators": the row step's input gradient is local, dY_i = dZ W2_i^T; the
// column step's is the shard's term of dX = sum_i dH_i W1_i^T).
struct BwdGemms {
  GemmArgs dh;        // dH = act'(H) * (dZ W2_i^T)            [T, s] (gated: [T, 2s])
  GemmArgs dw2;       // dW2_i = Y_i^T dZ                      [s, d]
  GemmArgs dx[2];     // dXp = dH W1_i^T (+ dU Wu_i^T)         [T, d]
  GemmArgs dw1[2];    // dW1_i = X^T dH (dWu_i = X^T dU)       [d, s]
  int n;              // weight-gradient GEMMs: 1, or 2 with SwiGLU
  int ndx;            // dX GEMMs: 1, or 2 with SwiGLU when the two terms cannot
                      // share one GEMM
};

BwdGemms bwd_gemms(const BwdCall &c) {
  const int64_t s = c.k / c.p, c0 = (int64_t)c.i * s;
  const size_t es = elem_size(c.dt);
  const bool gated = c.act == TP_ACT_SWIGLU;
  BwdGemms b{};
  b.n = gated ? 2 : 1;
  GemmArgs &h = b.dh;
  h.A = c.dZ;
  h.lda = c.lddz;
  h.B = (const char *)c.W2 + c0 * c.ldw2 * es;  // rows c0.. of W2 are the columns of W2_i^T
  h.ldb = c.ldw2;
  h.lay = LAY_NT;
  h.C = c.dH;
  h.ldc = c.lddh;
  h.aux = c.H;
  h.ldaux = c.ldh;
  h.M = c.T;
  h.N = s;
  h.K = c.d;
  h.epi = gated ? EPI_DSWIGLU : EPI_DACT;
  h.act = gated ? TP_ACT_SWIGLU : c.act;
  h.groups = 1;
  GemmArgs &w2 = b.dw2;
  w2.A = c.Y;  // held as Y_i [T, s] = (Y_i^T)^T
  w2.lda = c.ldy;
  w2.lay = LAY_TN;
  w2.B = c.dZ;
  w2.ldb = c.lddz;
  w2.C = c.dW2;
  w2.ldc = c.lddw2;
  w2.M = s;
  w2.N = c.d;
  w2.K = c.T;
  w2.epi = EPI_F32;
  w2.act = TP_ACT_NONE;
  w2.groups = 1;
  // With SwiGLU, dXp = dG Wg_i^T + dU Wu_i^T is one GEMM over K = 2s when the
  // two weights share a leading dimension and s is a whole number of k-steps:
  // dH = [dG | dU] is then A, and B^T's rows run through Wg_i then Wu_i.
  const bool fuse = gated && s % 32 == 0 && c.ldw1 == c.ldwu;
  b.ndx = gated && !fuse ? 2 : 1;
  for (int q = 0; q < b.n; ++q) {
    const void *Wq = q == 0 ? c.W1 : c.Wu;
    const int64_t ldwq = q == 0 ? c.ldw1 : c.ldwu;
    const void *dHq = (const char *)c.dH + q * s * es;
    if (q < b.ndx) {
      GemmArgs &x = b.dx[q];
      x.A = dHq;
      x.lda = c.lddh;
      x.B = (const char *)Wq + c0 * es;  // W_i^T: row n of W, columns c0..
      x.ldb = ldwq;
      x.lay = LAY_NT;
      x.C = c.dXp;
      x.ldc = c.lddx;
      x.M = c.T;
      x.N = c.d;
      x.K = s;
      x.epi = q == 0 ? EPI_F32 : EPI_F32_ACC;
      x.act = TP_ACT_NONE;
      x.groups = 1;
      if (fuse) {
        x.B2 = (const char *)c.Wu + c0 * es;
        x.ldb2 = c.ldwu;
        x.K = 2 * s;
        x.ksplit = s;
      }
    }
    GemmArgs &w = b.dw1[q];
    w.A = c.X;  // held as X [T, d] = (X^T)^T
    w.lda = c.ldx;
    w.lay = LAY_TN;
    w.B = dHq;
    w.ldb = c.lddh;
    w.C = q == 0 ? c.dW1 : c.dWu;
    w.ldc = q == 0 ? c.lddw1 : c.lddwu;
    w.M = c.d;
    w.N = s;
    w.K = c.T;
    w.epi = EPI_F32;
    w.act = TP_ACT_NONE;
    w.groups = 1;
  }
  return b;
}

// The bias gradient's column sums use the scratch part of the shared
// workspace layout (after the counter area), so one workspace buffer can
// serve the forward and backward entry points alike.
size_t bwd_ws_bytes(const BwdCall &c) {
  return c.db1 ? kWsCounterBytes + colsum_workspace_bytes(c.T, c.k / c.p) : 0;
}

QkvCall make_qkv(tp_dtype dt, int64_t T, int64_t d, int32_t Hq, int32_t Hkv, int64_t dh,
                 int32_t i, int32_t p, const void *X, int64_t ldx, const void *W, int64_t ldw,
                 const void *b, void *QKV, int64_t ldo) {
  QkvCall c;
  c.dt = dt;
  c.T = T;
  c.d = d;
  c.Hq = Hq;
  c.Hkv = Hkv;
  c.dh = dh;
  c.i = i;
  c.p = p;
  c.X = X;
  c.W = W;
  c.b = b;
  c.ldx = ldx;
  c.ldw = ldw;
  c.ldo = ldo;
  c.QKV = QKV;
  return c;
}

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of the simulated transformer block, in byte offsets: the counter
// area (and the few-token GEMMs' scratch) first, as for every entry point,
// then the block's own buffers.
struct BlockLayout {
  size_t a, qkv, o, y, x1, parts, total;
};
BlockLayout block_layout(size_t gemm_ws, int64_t T, int64_t d, int64_t nqkv, int64_t qw, int64_t s,
                         int32_t p) {
  BlockLayout L;
  size_t off = up256(max_sz(gemm_ws, kWsCounterBytes));
  L.a = off;
  off += up256((size_t)(T * d) * 2);
  L.qkv = off;
  off += up256((size_t)(T * nqkv) * 2);
  L.o = off;
  off += up256((size_t)(T * qw) * 2);
  L.y = off;
  off += up256((size_t)p * (size_t)(T * s) * 2);
  L.x1 = off;
  off += up256((size_t)(T * d) * 4);
  L.parts = off;
  off += up256((size_t)p * (size_t)(T * d) * 4);
  L.total = off;
  return L;
}

tp_status run_rownorm(const RowNormArgs &a, hipStream_t st) {
  const hipError_t e = launch_residual_ln(a, st);
  if (e != hipSuccess) return fail(TP_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return TP_OK;
}

tp_status check_eps(float eps) {
  if (!(eps >= 0.0f) || !__builtin_isfinite(eps))
    return fail(TP_ERR_BAD_SHAPE, "eps = %g must be finite and >= 0", (double)eps);
  return TP_OK;
}

// The GEMM descriptors of the simulated block and the workspace they and the
// block's buffers need; `ws` may be NULL for a size query.
struct BlockPlan {
  tp_status st;
  int64_t T, qw, nqkv, s;
  BlockLayout L;
  size_t gemm_ws;
};
BlockPlan plan_block(tp_dtype dt, tp_act act, int64_t nseq, int64_t S, int64_t d, int32_t Hq,
                     int32_t Hkv, int64_t dh, int64_t k, int32_t p) {
  BlockPlan P{};
  P.st = TP_OK;
  auto bad = [&](tp_status st) {
    P.st = st;
    return P;
  };
  if (dt != TP_BF16)
    return bad(fail(TP_ERR_BAD_DTYPE, "the transformer block runs in bf16 only (dtype %d)",
                    (int)dt));
  if (check_dtype_act(dt, act) != TP_OK) return bad(TP_ERR_BAD_ACT);
  if (nseq < 0 || S < 0)
    return bad(fail(TP_ERR_BAD_SHAPE, "nseq = %lld and S = %lld must be >= 0", (long long)nseq,
                    (long long)S));
  if (d < 8 || d > kRowNormMaxD || d % 8)
    return bad(fail(d % 8 ? TP_ERR_MISALIGNED : TP_ERR_BAD_SHAPE,
                    "d = %lld must be a multiple of 8 in [8, %lld]", (long long)d,
                    (long long)kRowNormMaxD));
  if (Hq < 1 || Hkv < 1)
    return bad(fail(TP_ERR_BAD_SHAPE, "Hq = %d and Hkv = %d must be >= 1", Hq, Hkv));
  if (Hq % Hkv)
    return bad(fail(TP_ERR_NOT_DIVISIBLE, "Hq = %d is not a multiple of Hkv = %d", Hq, Hkv));
  if (dh != 64 && dh != 128)
    return bad(fail(TP_ERR_BAD_SHAPE, "head width dh = %lld: 64 and 128 are supported",
                    (long long)dh));
  if (p < 1 || p > TP_MAX_SHARDS)
    return bad(fail(TP_ERR_BAD_SHARD, "p = %d outside [1, %d]", p, TP_MAX_SHARDS));
  if (Hq % p || Hkv % p || k < 1 || k % p)
    return bad(fail(TP_ERR_NOT_DIVISIBLE, "Hq = %d, Hkv = %d and k = %lld must be divisible by p = %d",
                    Hq, Hkv, (long long)k, p));
  if (nseq > 0 && S > (int64_t(1) << 40) / nseq)
    return bad(fail(TP_ERR_BAD_SHAPE, "nseq * S is too large"));
  P.T = nseq * S;
  P.qw = (int64_t)Hq * dh / p;  // one shard's attention-output columns (W_O rows)
  P.nqkv = ((int64_t)Hq + 2 * (int64_t)Hkv) * dh;  // all shards' QKV columns
  P.s = k / p;
  // Scratch of the GEMMs (split-K partials: the few-token path's, or the
  // tiled path's for shapes with few tiles): the largest of the block's four
  // GEMM shapes; buffers are placeholders here.
  static const char dummy[16] __attribute__((aligned(16))) = {0};
  const int64_t T = P.T;
  const QkvCall qc = make_qkv(dt, T, d, Hq, Hkv, dh, 0, 1, dummy, d, dummy, P.nqkv, nullptr,
                              (void *)dummy, P.nqkv);
  const RowCall ro = make_row(dt, T, d, (int64_t)Hq * dh, 0, p, dummy, (int64_t)Hq * dh, dummy,
                              d, (float *)dummy, d);
  const ColCall c = make_col(dt, act, T, d, k, 0, p, dummy, d, dummy, k, dummy, k, nullptr,
                             (void *)dummy, P.s);
  const RowCall r = make_row(dt, T, d, k, 0, p, dummy, P.s, dummy, d, (float *)dummy, d);
  size_t g = gemm_ws_bytes(dt, qkv_gemm(qc));
  g = max_sz(g, gemm_ws_bytes(dt, row_gemm(ro, p, P.qw, T * d)));
  g = max_sz(g, gemm_ws_bytes(dt, col_gemm(c, p, T * P.s)));
  g = max_sz(g, gemm_ws_bytes(dt, row_gemm(r, p, T * P.s, T * d)));
  P.gemm_ws = g;
  P.L = block_layout(g, T, d, P.nqkv, (int64_t)Hq * dh, P.s, p);
  return P;
}
}  // namespace

extern "C" {

tp_status tp_col_linear(tp_dtype dt, tp_act act, int64_t T, int64_t d, int64_t k, int32_t i,
                        int32_t p, const void *X, int64_t ldx, const void *W1, int64_t ldw1,
                        const void *Wu, int64_t ldwu, const void *b1, void *Y, int64_t ldy,
                        void *ws, size_t ws_bytes, void *stream) {
  const ColCall c = make_col(dt, act, T, d, k, i, p, X, ldx, W1, ldw1, Wu, ldwu, b1, Y, ldy);
  TRY(validate_col(c));
  if (T == 0) return ok();
  GemmArgs a = col_gemm(c, 1, 0);
  TRY(check_gemm(dt, a));
  TRY(check_ws(fit_gemm_ws(dt, a, ws, ws_bytes), ws, ws_bytes));
  TRY(run_gemm(dt, a, ws, (hipStream_t)stream));
  return ok();
}

tp_status tp_row_linear(tp_dtype dt, int64_t T, int64_t d, int64_t k, int32_t i, int32_t p,
                        const void *Y, int64_t ldy, const void *W2, int64_t ldw2, float *Z,
                        int64_t ldz, void *ws, size_t ws_bytes, void *stream) {
  const RowCall r = make_row(dt, T, d, k, i, p, Y, ldy, W2, ldw2, Z, ldz);
  TRY(validate_row(r));
  if (T == 0) return ok();
  GemmArgs a = row_gemm(r, 1, 0, 0);
  TRY(check_gemm(dt, a));
  TRY(check_ws(fit_gemm_ws(dt, a, ws, ws_bytes), ws, ws_bytes));
  TRY(run_gemm(dt, a, ws, (hipStream_t)stream));
  return ok();
}

tp_status tp_mlp_shard(tp_dtype dt, tp_act act, int64_t T, int64_t d, int64_t k, int32_t i,
                       int32_t p, const void *X, int64_t ldx, const void *W1, int64_t ldw1,
                       const void *Wu, int64_t ldwu, const void *b1, const void *W2,
                       int64_t ldw2, void *Y, int64_t ldy, float *Z, int64_t ldz, void *ws,
                       size_t ws_bytes, void *stream) {
  const ColCall c = make_col(dt, act, T, d, k, i, p, X, ldx, W1, ldw1, Wu, ldwu, b1, Y, ldy);
  TRY(validate_col(c));
  const RowCall r = make_row(dt, T, d, k, i, p, Y, ldy, W2, ldw2, Z, ldz);
  TRY(validate_row(r));
  if (T == 0) return ok();
  GemmArgs ac = col_gemm(c, 1, 0), ar = row_gemm(r, 1, 0, 0);
  TRY(check_gemm(dt, ac));
  TRY(check_gemm(dt, ar));
  TRY(check_ws(max_sz(fit_gemm_ws(dt, ac, ws, ws_bytes), fit_gemm_ws(dt, ar, ws, ws_bytes)), ws,
               ws_bytes));
  TRY(run_gemm(dt, ac, ws, (hipStream_t)stream));
  TRY(run_gemm(dt, ar, ws, (hipStream_t)stream));
  return ok();
}

tp_status tp_mlp_shard_noalloc(tp_dtype dt, tp_act act, int64_t T, int64_t d, int64_t k, int32_t i,
                               int32_t p, const void *X, int64_t ldx, const void *W1,
                               int64_t ldw1, const void *Wu, int64_t ldwu, const void *b1,
                               const void *W2, int64_t ldw2, void *Y, int64_t ldy, float *Z,
                               int64_t ldz, void *stream) {
  static_assert(kStaticScratchBytes == TP_STATIC_SCRATCH_BYTES, "scratch size");
  const ColCall c = make_col(dt, act, T, d, k, i, p, X, ldx, W1, ldw1, Wu, ldwu, b1, Y, ldy);
  TRY(validate_col(c));
  const RowCall r = make_row(dt, T, d, k, i, p, Y, ldy, W2, ldw2, Z, ldz);
  TRY(validate_row(r));
  if (T == 0) return ok();
  // The tiled path's split-K partials would not fit the static scratch: the
  // many-token GEMMs run unsplit here.
  GemmArgs ac = col_gemm(c, 1, 0), ar = row_gemm(r, 1, 0, 0);
  ac.splitk = ar.splitk = 1;
  TRY(check_gemm(dt, ac));
  TRY(check_gemm(dt, ar));
  const size_t need = max_sz(gemm_ws_bytes(dt, ac), gemm_ws_bytes(dt, ar));
  if (need > kStaticScratchBytes)
    return fail(TP_ERR_WORKSPACE,
                "these sizes need %zu bytes of scratch; the static scratch holds %zu", need,
                kStaticScratchBytes);
  void *ws = nullptr;
  if (need > 0) {
    const hipError_t e = static_scratch((hipStream_t)stream, &ws);
    if (e != hipSuccess)
      return fail(TP_ERR_HIP, "static scratch set-up failed: %s", hipGetErrorString(e));
  }
  TRY(run_gemm(dt, ac, ws, (hipStream_t)stream));
  TRY(run_gemm(dt, ar, ws, (hipStream_t)stream));
  return ok();
}

tp_status tp_partial_sum(int64_t T, int64_t d, int32_t p, const float *const *parts, int64_t ldp,
                         const float *b2, float *Z, int64_t ldz, void *stream) {
  if (T < 0) return fail(TP_ERR_BAD_SHAPE, "T = %lld < 0", (long long)T);
  if (d < 1) return fail(TP_ERR_BAD_SHAPE, "d = %lld < 1", (long long)d);
  if (p < 1 || p > TP_MAX_SHARDS)
    return fail(TP_ERR_BAD_SHARD, "p = %d outside [1, %d]", p, TP_MAX_SHARDS);
  if (d % 4) return fail(TP_ERR_MISALIGNED, "d = %lld is not a multiple of 4", (long long)d);
  if (!parts) return fail(TP_ERR_NULL_POINTER, "parts is NULL");
  TRY(check_ld("ldp", ldp, d, TP_F32));
  TRY(check_ld("ldz", ldz, d, TP_F32));
  if (T == 0) return ok();  // nothing is read or written
  PartSumArgs a{};
  for (int q = 0; q < p; ++q) {
    char name[32];
    snprintf(name, sizeof name, "parts[%d]", q);
    TRY(check_ptr(name, parts[q]));
    a.parts[q] = parts[q];
  }
  TRY(check_ptr("Z", Z));
  if (b2) TRY(check_ptr("b2", b2));
  a.p = p;
  a.T = T;
  a.d = d;
  a.ldp = ldp;
  a.ldz = ldz;
  a.b2 = b2;
  a.Z = Z;
  const hipError_t e = launch_partial_sum(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TP_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

tp_status tp_mlp_simulated(tp_dtype dt, tp_act act, int64_t T, int64_t d, int64_t k, int32_t p,
                           const void *X, int64_t ldx, const void *W1, int64_t ldw1,
                           const void *Wu, int64_t ldwu, const void *b1, const void *W2,
                           int64_t ldw2, const float *b2, void *Y, float *Zp, float *Z,
                           int64_t ldz, void *ws, size_t ws_bytes, void *stream) {
  if (p < 1 || p > TP_MAX_SHARDS)
    return fail(TP_ERR_BAD_SHARD, "p = %d outside [1, %d]", p, TP_MAX_SHARDS);
  const int64_t s = (p > 0 && k % p == 0) ? k / p : 0;
  // Shard 0 stands for all: the others differ only by the block offsets.
  const ColCall c = make_col(dt, act, T, d, k, 0, p, X, ldx, W1, ldw1, Wu, ldwu, b1, Y, s);
  TRY(validate_col(c));
  const RowCall r = make_row(dt, T, d, k, 0, p, Y, s, W2, ldw2, Zp, d);
  TRY(validate_row(r));
  if (T > 0) TRY(check_ptr("Z", Z));
  TRY(check_ld("ldz", ldz, d, TP_F32));
  if (b2) TRY(check_ptr("b2", b2));
  if (T == 0) return ok();
  GemmArgs ac = col_gemm(c, p, T * s), ar = row_gemm(r, p, T * s, T * d);
  TRY(check_gemm(dt, ac));
  TRY(check_gemm(dt, ar));
  TRY(check_ws(max_sz(fit_gemm_ws(dt, ac, ws, ws_bytes), fit_gemm_ws(dt, ar, ws, ws_bytes)), ws,
               ws_bytes));
  TRY(run_gemm(dt, ac, ws, (hipStream_t)stream));
  TRY(run_gemm(dt, ar, ws, (hipStream_t)stream));
  PartSumArgs ps{};
  for (int q = 0; q < p; ++q) ps.parts[q] = Zp + (int64_t)q * T * d;
  ps.p = p;
  ps.T = T;
  ps.d = d;
  ps.ldp = d;
  ps.ldz = ldz;
  ps.b2 = b2;
  ps.Z = Z;
  const hipError_t e = launch_partial_sum(ps, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TP_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t tp_workspace_bytes(tp_dtype dt, tp_act act, int64_t T, int64_t d, int64_t k, int32_t p) {
  if (dt != TP_F32 && dt != TP_BF16) return 0;
  if ((int)act < TP_ACT_NONE || (int)act > TP_ACT_SWIGLU) return 0;
  if (T < 1 || d < 1 || k < 1 || p < 1 || p > TP_MAX_SHARDS || k % p) return 0;
  const int64_t s = k / p;
  static const char dummy[16] __attribute__((aligned(16))) = {0};
  ColCall c = make_col(dt, act, T, d, k, 0, p, dummy, d, dummy, k, dummy, k, nullptr,
                       (void *)dummy, s);
  RowCall r = make_row(dt, T, d, k, 0, p, dummy, s, dummy, d, (float *)dummy, d);
  // One shard (tp_col_linear, tp_row_linear, tp_mlp_shard) and all p shards
  // as grouped launches (tp_mlp_simulated): the split may differ.
  size_t need = max_sz(gemm_ws_bytes(dt, col_gemm(c, 1, 0)), gemm_ws_bytes(dt, row_gemm(r, 1, 0, 0)));
  need = max_sz(need, gemm_ws_bytes(dt, col_gemm(c, p, T * s)));
  return max_sz(need, gemm_ws_bytes(dt, row_gemm(r, p, T * s, T * d)));
}

tp_status tp_col_linear_train(tp_dtype dt, tp_act act, int64_t T, int64_t d, int64_t k, int32_t i,
                              int32_t p, const void *X, int64_t ldx, const void *W1, int64_t ldw1,
                              const void *Wu, int64_t ldwu, const void *b1, void *Y, int64_t ldy,
                              void *H, int64_t ldh, void *stream) {
  const ColCall c = make_col(dt, act, T, d, k, i, p, X, ldx, W1, ldw1, Wu, ldwu, b1, Y, ldy);
  TRY(validate_col(c));
  const int64_t s = (k / p) * (act == TP_ACT_SWIGLU ? 2 : 1);
  if (T > 0) TRY(check_ptr("H", H));
  TRY(check_ld("ldh", ldh, s, dt));
  if (T == 0) return ok();
  GemmArgs a = col_gemm(c, 1, 0);
  a.epi = act == TP_ACT_SWIGLU ? EPI_SWIGLU_SAVE : EPI_ACT_SAVE;
  a.C2 = H;
  a.ldc2 = ldh;
  TRY(check_tiled(dt, a));
  TRY(run_tiled(dt, a, (hipStream_t)stream));
  return ok();
}

tp_status tp_mlp_shard_backward(tp_dtype dt, tp_act act, int64_t T, int64_t d, int64_t k, int32_t i,
                                int32_t p, const void *X, int64_t ldx, const void *W1, int64_t ldw1,
                                const void *Wu, int64_t ldwu, const void *W2, int64_t ldw2,
                                const void *H, int64_t ldh, const void *Y, int64_t ldy,
                                const void *dZ, int64_t lddz, void *dH, int64_t lddh, float *dXp,
                                int64_t lddx, float *dW1, int64_t lddw1, float *dWu, int64_t lddwu,
                                float *db1, float *dW2, int64_t lddw2, void *ws, size_t ws_bytes,
                                void *stream) {
  BwdCall c;
  c.dt = dt;
  c.act = (int)act;
  c.T = T;
  c.d = d;
  c.k = k;
  c.i = i;
  c.p = p;
  c.X = X;
  c.W1 = W1;
  c.Wu = act == TP_ACT_SWIGLU ? Wu : nullptr;
  c.W2 = W2;
  c.H = H;
  c.Y = Y;
  c.dZ = dZ;
  c.ldx = ldx;
  c.ldw1 = ldw1;
  c.ldwu = ldwu;
  c.ldw2 = ldw2;
  c.ldh = ldh;
  c.ldy = ldy;
  c.lddz = lddz;
  c.dH = dH;
  c.lddh = lddh;
  c.dXp = dXp;
  c.dW1 = dW1;
  c.dWu = act == TP_ACT_SWIGLU ? dWu : nullptr;
  c.db1 = db1;
  c.dW2 = dW2;
  c.lddx = lddx;
  c.lddw1 = lddw1;
  c.lddwu = lddwu;
  c.lddw2 = lddw2;
  TRY(validate_bwd(c));
  const BwdGemms b = bwd_gemms(c);
  TRY(check_tiled(dt, b.dh));
  TRY(check_tiled(dt, b.dw2));
  for (int q = 0; q < b.ndx; ++q) TRY(check_tiled(dt, b.dx[q]));
  for (int q = 0; q < b.n; ++q) TRY(check_tiled(dt, b.dw1[q]));
  TRY(check_ws(bwd_ws_bytes(c), ws, ws_bytes));
  const hipStream_t st = (hipStream_t)stream;
  // With no tokens the weight and bias gradients are zero: the weight-gradient
  // GEMMs (K = T = 0) and the column sum write zeros; the others launch nothing.
  TRY(run_tiled(dt, b.dh, st));
  TRY(run_tiled(dt, b.dw2, st));
  for (int q = 0; q < b.ndx; ++q) TRY(run_tiled(dt, b.dx[q], st));
  for (int q = 0; q < b.n; ++q) TRY(run_tiled(dt, b.dw1[q], st));
  if (db1) {
    const hipError_t e = launch_colsum(dt == TP_BF16, dH, lddh, T, k / p,
                                       (float *)((char *)ws + kWsCounterBytes), db1, st);
    if (e != hipSuccess) return fail(TP_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  }
  return ok();
}

size_t tp_backward_workspace_bytes(tp_dtype dt, tp_act act, int64_t T, int64_t d, int64_t k,
                                   int32_t p, int32_t with_db1) {
  if (dt != TP_F32 && dt != TP_BF16) return 0;
  if ((int)act < TP_ACT_NONE || (int)act > TP_ACT_SWIGLU) return 0;
  if (T < 0 || d < 1 || k < 1 || p < 1 || p > TP_MAX_SHARDS || k % p) return 0;
  if (!with_db1 || act == TP_ACT_SWIGLU) return 0;
  return kWsCounterBytes + colsum_workspace_bytes(T, k / p);
}

tp_status tp_qkv_linear(tp_dtype dt, int64_t T, int64_t d, int32_t Hq, int32_t Hkv, int64_t dh,
                        int32_t i, int32_t p, const void *X, int64_t ldx, const void *Wqkv,
                        int64_t ldw, const void *bqkv, void *QKV, int64_t ldo, void *ws,
                        size_t ws_bytes, void *stream) {
  const QkvCall c = make_qkv(dt, T, d, Hq, Hkv, dh, i, p, X, ldx, Wqkv, ldw, bqkv, QKV, ldo);
  TRY(validate_qkv(c));
  if (T == 0) return ok();
  GemmArgs a = qkv_gemm(c);
  TRY(check_gemm(dt, a));
  TRY(check_ws(fit_gemm_ws(dt, a, ws, ws_bytes), ws, ws_bytes));
  TRY(run_gemm(dt, a, ws, (hipStream_t)stream));
  return ok();
}

tp_status tp_attention(tp_dtype dt, int64_t nseq, int64_t S, int32_t Hq, int32_t Hkv, int64_t dh,
                       int32_t causal, const void *Q, int64_t ldq, const void *K, int64_t ldk,
                       const void *V, int64_t ldv, void *O, int64_t ldo, void *stream) {
  if (dt != TP_BF16)
    return fail(TP_ERR_BAD_DTYPE, "the attention core runs in bf16 only (dtype %d)", (int)dt);
  if (nseq < 0 || S < 0)
    return fail(TP_ERR_BAD_SHAPE, "nseq = %lld and S = %lld must be >= 0", (long long)nseq,
                (long long)S);
  if (Hq < 1 || Hkv < 1)
    return fail(TP_ERR_BAD_SHAPE, "Hq = %d and Hkv = %d must be >= 1", Hq, Hkv);
  if (Hq % Hkv)
    return fail(TP_ERR_NOT_DIVISIBLE, "Hq = %d is not a multiple of Hkv = %d", Hq, Hkv);
  if (dh != 64 && dh != 128)
    return fail(TP_ERR_BAD_SHAPE, "head width dh = %lld: 64 and 128 are supported", (long long)dh);
  TRY(check_ld("ldq", ldq, (int64_t)Hq * dh, dt));
  TRY(check_ld("ldk", ldk, (int64_t)Hkv * dh, dt));
  TRY(check_ld("ldv", ldv, (int64_t)Hkv * dh, dt));
  TRY(check_ld("ldo", ldo, (int64_t)Hq * dh, dt));
  if (nseq == 0 || S == 0) return ok();
  TRY(check_ptr("Q", Q));
  TRY(check_ptr("K", K));
  TRY(check_ptr("V", V));
  TRY(check_ptr("O", O));
  AttnArgs a{};
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  a.ldq = ldq;
  a.ldk = ldk;
  a.ldv = ldv;
  a.ldo = ldo;
  a.nseq = nseq;
  a.S = S;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.dh = (int)dh;
  a.causal = causal ? 1 : 0;
  a.scale_log2 = (float)(1.4426950408889634 / __builtin_sqrt((double)dh));
  if (!attention_supported(a))
    return fail(TP_ERR_BAD_SHAPE, "leading dimensions must be below 2^23 elements");
  const hipError_t e = launch_attention(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TP_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t tp_qkv_workspace_bytes(tp_dtype dt, int64_t T, int64_t d, int32_t Hq, int32_t Hkv,
                              int64_t dh, int32_t p) {
  static const char dummy[16] __attribute__((aligned(16))) = {0};
  if (T < 1 || d < 1 || Hq < 1 || Hkv < 1 || dh < 1 || p < 1 || p > TP_MAX_SHARDS) return 0;
  const int64_t ncol = ((int64_t)Hq + 2 * (int64_t)Hkv) * dh;
  const QkvCall c = make_qkv(dt, T, d, Hq, Hkv, dh, 0, p, dummy, d, dummy, ncol, nullptr,
                             (void *)dummy, p > 0 ? ncol / p : ncol);
  const std::string keep = g_msg;  // a size query leaves the last error message alone
  const tp_status st = validate_qkv(c);
  g_msg = keep;
  if (st != TP_OK) return 0;
  return gemm_ws_bytes(dt, qkv_gemm(c));
}

tp_status tp_residual_layernorm(int64_t T, int64_t d, int32_t p, const float *const *parts,
                                int64_t ldp, const float *bias, const float *R, int64_t ldr,
                                float *X, int64_t ldx, const float *gamma, const float *beta,
                                float eps, void *A, int64_t lda, void *stream) {
  if (T < 0) return fail(TP_ERR_BAD_SHAPE, "T = %lld < 0", (long long)T);
  if (d < 1 || d > kRowNormMaxD)
    return fail(TP_ERR_BAD_SHAPE, "d = %lld outside [1, %lld]", (long long)d,
                (long long)kRowNormMaxD);
  if (d % 8) return fail(TP_ERR_MISALIGNED, "d = %lld is not a multiple of 8", (long long)d);
  if (p < 0 || p > TP_MAX_SHARDS)
    return fail(TP_ERR_BAD_SHARD, "p = %d outside [0, %d]", p, TP_MAX_SHARDS);
  if (p > 0 && !parts) return fail(TP_ERR_NULL_POINTER, "parts is NULL");
  TRY(check_eps(eps));
  if (p > 0) TRY(check_ld("ldp", ldp, d, TP_F32));
  if (R) TRY(check_ld("ldr", ldr, d, TP_F32));
  if (X) TRY(check_ld("ldx", ldx, d, TP_F32));
  if (A) TRY(check_ld("lda", lda, d, TP_BF16));
  if (T == 0) return ok();  // nothing is read or written; buffers may be NULL
  if (p == 0 && !bias && !R)
    return fail(TP_ERR_BAD_SHAPE, "nothing to add: no partials, no bias and no residual");
  if (!X && !A) return fail(TP_ERR_BAD_SHAPE, "no output: X and A are both NULL");
  if ((gamma != nullptr) != (A != nullptr) || (gamma != nullptr) != (beta != nullptr))
    return fail(TP_ERR_NULL_POINTER, "gamma, beta and A are given together or not at all");
  RowNormArgs a{};
  for (int q = 0; q < p; ++q) {
    char name[32];
    snprintf(name, sizeof name, "parts[%d]", q);
    TRY(check_ptr(name, parts[q]));
    a.parts[q] = parts[q];
  }
  if (bias) TRY(check_ptr("bias", bias));
  if (R) TRY(check_ptr("R", R));
  if (X) TRY(check_ptr("X", X));
  if (A) {
    TRY(check_ptr("gamma", gamma));
    TRY(check_ptr("beta", beta));
    TRY(check_ptr("A", A));
  }
  a.p = p;
  a.T = T;
  a.d = d;
  a.ldp = ldp;
  a.bias = bias;
  a.R = R;
  a.ldr = ldr;
  a.X = X;
  a.ldx = ldx;
  a.gamma = gamma;
  a.beta = beta;
  a.eps = eps;
  a.A = A;
  a.lda = lda;
  TRY(run_rownorm(a, (hipStream_t)stream));
  return ok();
}

size_t tp_block_workspace_bytes(tp_dtype dt, tp_act act, int64_t nseq, int64_t S, int64_t d,
                                int32_t Hq, int32_t Hkv, int64_t dh, int64_t k, int32_t p) {
  const std::string keep = g_msg;  // a size query leaves the last error message alone
  const BlockPlan P = plan_block(dt, act, nseq, S, d, Hq, Hkv, dh, k, p);
  g_msg = keep;
  if (P.st != TP_OK || P.T == 0) return 0;
  return P.L.total;
}

tp_status tp_block_simulated(tp_dtype dt, tp_act act, int64_t nseq, int64_t S, int64_t d,
                             int32_t Hq, int32_t Hkv, int64_t dh, int64_t k, int32_t p,
                             int32_t causal, float eps, const float *X, int64_t ldx,
                             const float *ln1_g, const float *ln1_b, const void *Wqkv,
                             int64_t ldwqkv, const void *bqkv, const void *WO, int64_t ldwo,
                             const float *bO, const float *ln2_g, const float *ln2_b,
                             const void *W1, int64_t ldw1, const void *Wu, int64_t ldwu,
                             const void *b1, const void *W2, int64_t ldw2, const float *b2,
                             float *Out, int64_t ldout, void *ws, size_t ws_bytes, void *stream) {
  const BlockPlan P = plan_block(dt, act, nseq, S, d, Hq, Hkv, dh, k, p);
  if (P.st != TP_OK) return P.st;
  const int64_t T = P.T;
  TRY(check_eps(eps));
  TRY(check_ptr("ln1_gamma", ln1_g));
  TRY(check_ptr("ln1_beta", ln1_b));
  TRY(check_ptr("ln2_gamma", ln2_g));
  TRY(check_ptr("ln2_beta", ln2_b));
  if (bO) TRY(check_ptr("bO", bO));
  if (b2) TRY(check_ptr("b2", b2));
  TRY(check_ld("ldx", ldx, d, TP_F32));
  TRY(check_ld("ldout", ldout, d, TP_F32));
  if (T > 0) {
    TRY(check_ptr("X", X));
    TRY(check_ptr("Out", Out));
  }
  // In this simulated mode the p shards' column blocks of the QKV projection
  // together are the whole projection: one GEMM computes all of them (every
  // output element is the same dot product, in the same order, as in the
  // shard's own launch), the attention core runs over all heads at once
  // (heads never mix), and the W_O row blocks are one grouped launch that
  // writes one fp32 partial per shard; likewise the FFN shards.  The checks
  // run on the real buffers once the workspace is known, or on placeholders
  // when there are no tokens.
  static const char dummy[16] __attribute__((aligned(16))) = {0};
  const BlockLayout &L = P.L;
  if (T > 0) TRY(check_ws(L.total, ws, ws_bytes));
  char *w = T > 0 ? (char *)ws : (char *)dummy;
  QkvCall qc = make_qkv(dt, T, d, Hq, Hkv, dh, 0, 1, dummy, d, Wqkv, ldwqkv, bqkv,
                        (void *)dummy, P.nqkv);
  ColCall c = make_col(dt, act, T, d, k, 0, p, dummy, d, W1, ldw1, Wu, ldwu, b1, (void *)dummy,
                       P.s);
  RowCall ro = make_row(dt, T, d, (int64_t)Hq * dh, 0, p, dummy, (int64_t)Hq * dh, WO, ldwo,
                        (float *)dummy, d);
  RowCall r = make_row(dt, T, d, k, 0, p, dummy, P.s, W2, ldw2, (float *)dummy, d);
  if (T > 0) {
    qc.X = w + L.a;
    qc.QKV = w + L.qkv;
    c.X = w + L.a;
    c.Y = w + L.y;
    ro.Y = w + L.o;
    ro.Z = (float *)(w + L.parts);
    r.Y = w + L.y;
    r.Z = (float *)(w + L.parts);
  }
  TRY(validate_qkv(qc));
  TRY(validate_col(c));
  TRY(validate_row(ro));
  TRY(validate_row(r));
  if (T == 0) return ok();
  const hipStream_t st = (hipStream_t)stream;
  float *parts = (float *)(w + L.parts);
  float *X1 = (float *)(w + L.x1);
  AttnArgs at{};
  at.nseq = nseq;
  at.S = S;
  at.Hq = Hq;
  at.Hkv = Hkv;
  at.dh = (int)dh;
  at.causal = causal ? 1 : 0;
  at.scale_log2 = (float)(1.4426950408889634 / __builtin_sqrt((double)dh));
  at.Q = w + L.qkv;
  at.K = w + L.qkv + (int64_t)Hq * dh * 2;
  at.V = w + L.qkv + ((int64_t)Hq + Hkv) * dh * 2;
  at.O = w + L.o;
  at.ldq = at.ldk = at.ldv = P.nqkv;
  at.ldo = (int64_t)Hq * dh;
  if (!attention_supported(at))
    return fail(TP_ERR_BAD_SHAPE, "attention shape beyond the kernel's range");
  const GemmArgs qg = qkv_gemm(qc), og = row_gemm(ro, p, P.qw, T * d);
  TRY(check_gemm(dt, qg));
  TRY(check_gemm(dt, og));
  const GemmArgs cg = col_gemm(c, p, T * P.s), rg = row_gemm(r, p, T * P.s, T * d);
  TRY(check_gemm(dt, cg));
  TRY(check_gemm(dt, rg));

  // A = LN1(X)
  RowNormArgs n1{};
  n1.p = 0;
  n1.T = T;
  n1.d = d;
  n1.R = X;
  n1.ldr = ldx;
  n1.gamma = ln1_g;
  n1.beta = ln1_b;
  n1.eps = eps;
  n1.A = w + L.a;
  n1.lda = d;
  TRY(run_rownorm(n1, st));
  // Attention of all shards: QKV, the core over every head, the W_O row blocks.
  TRY(run_gemm(dt, qg, ws, st));
  const hipError_t e = launch_attention(at, st);
  if (e != hipSuccess) return fail(TP_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  TRY(run_gemm(dt, og, ws, st));
  // X1 = sum of the partials + bO + X;  A = LN2(X1)
  RowNormArgs n2{};
  for (int32_t i = 0; i < p; ++i) n2.parts[i] = parts + (int64_t)i * T * d;
  n2.p = p;
  n2.T = T;
  n2.d = d;
  n2.ldp = d;
  n2.bias = bO;
  n2.R = X;
  n2.ldr = ldx;
  n2.X = X1;
  n2.ldx = d;
  n2.gamma = ln2_g;
  n2.beta = ln2_b;
  n2.eps = eps;
  n2.A = w + L.a;
  n2.lda = d;
  TRY(run_rownorm(n2, st));
  // The FFN of all p shards (grouped launches), then Out = sum + b2 + X1.
  TRY(run_gemm(dt, cg, ws, st));
  TRY(run_gemm(dt, rg, ws, st));
  RowNormArgs n3{};
  for (int32_t i = 0; i < p; ++i) n3.parts[i] = parts + (int64_t)i * T * d;
  n3.p = p;
  n3.T = T;
  n3.d = d;
  n3.ldp = d;
  n3.bias = b2;
  n3.R = X1;
  n3.ldr = d;
  n3.X = Out;
  n3.ldx = ldout;
  TRY(run_rownorm(n3, st));
  return ok();
}

tp_status tp_shard_bounds(int64_t k, int32_t i, int32_t p, int64_t *c0, int64_t *s) {
  if (!c0 || !s) return fail(TP_ERR_NULL_POINTER, "output pointer is NULL");
  TRY(check_shard(0, 1, k, i, p));
  *s = k / p;
  *c0 = (int64_t)i * (k / p);
  return ok();
}

const char *tp_status_string(tp_status s) {
  switch (s) {
    case TP_OK:
      return "TP_OK";
    case TP_ERR_NULL_POINTER:
      return "TP_ERR_NULL_POINTER";
    case TP_ERR_BAD_SHAPE:
      return "TP_ERR_BAD_SHAPE";
    case TP_ERR_NOT_DIVISIBLE:
      return "TP_ERR_NOT_DIVISIBLE";
    case TP_ERR_BAD_SHARD:
      return "TP_ERR_BAD_SHARD";
    case TP_ERR_MISALIGNED:
      return "TP_ERR_MISALIGNED";
    case TP_ERR_BAD_DTYPE:
      return "TP_ERR_BAD_DTYPE";
    case TP_ERR_BAD_ACT:
      return "TP_ERR_BAD_ACT";
    case TP_ERR_WORKSPACE:
      return "TP_ERR_WORKSPACE";
    case TP_ERR_HIP:
      return "TP_ERR_HIP";
  }
  return "TP_UNKNOWN_STATUS";
}

const char *tp_last_error_message(void) { return g_msg.c_str(); }

int32_t tp_abi_version(void) { return TPMLP_ABI_VERSION; }

}  // extern "C"

extern "C" tp_status tp_calib_mfma_bf16(int32_t gaussian, int64_t iters, uint64_t *stats,
                                        int32_t nwg, void *stream) {
  if (nwg < 1 || iters < 1)
    return fail(TP_ERR_BAD_SHAPE, "nwg = %d and iters = %lld must be >= 1", nwg, (long long)iters);
  if (!stats) return fail(TP_ERR_NULL_POINTER, "stats is NULL");
  const hipError_t e = launch_calib_mfma(gaussian ? 1 : 0, iters, stats, nwg, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TP_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

extern "C" tp_status tp_calib_hbm_read(const void *buf, int64_t bytes, uint32_t *sink, int32_t nwg,
                                       void *stream) {
  if (nwg < 1 || bytes < 0 || bytes % 16)
    return fail(TP_ERR_BAD_SHAPE, "nwg = %d must be >= 1 and bytes = %lld a multiple of 16", nwg,
                (long long)bytes);
  if (!sink) return fail(TP_ERR_NULL_POINTER, "sink is NULL");
  if (bytes > 0) TRY(check_ptr("buf", buf));
  if (bytes == 0) return ok();
  const hipError_t e = launch_calib_hbm_read(buf, bytes, sink, nwg, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TP_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}
