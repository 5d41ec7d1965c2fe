// Calls libtpmlp's C ABI on fake device buffers, one case per input line, and
// reports what the bounds model found (test infrastructure, CPU only).
//
//   driver < cases.txt
//
// A case line is an entry point and its sizes; a leading '!' marks a call that
// must be rejected (a status other than TP_OK and no launch).  Every operand
// gets a buffer of exactly the bytes its documented shape needs, so that an
// access past the last element of any operand is a finding.  One output line
// per case:
//   CASE <line> | status <s> launches <n> tiled <n> decode <n> other <n> accesses <n> findings <n>
// followed by a FINDING line for each finding.  Exit status 0 when every case
// returned the expected status and nothing was found.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <map>
#include <sstream>
#include <string>
#include <vector>

#include "../../include/tpmlp.h"
#include "model.hpp"

namespace {

using hostcheck::fake_alloc;

int64_t es_of(tp_dtype dt) { return dt == TP_BF16 ? 2 : 4; }

// Bytes of a [rows, cols] matrix with leading dimension ld (0 rows: 1 byte, so
// that the pointer is still a valid, registered address).
size_t mat(int64_t rows, int64_t cols, int64_t ld, int64_t es) {
  if (rows <= 0 || cols <= 0) return 16;
  return (size_t)(((rows - 1) * ld + cols) * es);
}

// Bytes taken off every buffer (a self-test of the model: the last elements
// of the operands then lie outside their buffers).
size_t g_shrink = 0;

void *buf(size_t bytes, const char *name) {
  if (bytes == 0) bytes = 16;
  return fake_alloc(bytes > g_shrink ? bytes - g_shrink : bytes, name);
}

tp_dtype parse_dt(const std::string &s) { return s == "f32" ? TP_F32 : TP_BF16; }

tp_act parse_act(const std::string &s) {
  if (s == "none") return TP_ACT_NONE;
  if (s == "relu") return TP_ACT_RELU;
  if (s == "gelu_tanh") return TP_ACT_GELU_TANH;
  if (s == "gelu_erf") return TP_ACT_GELU_ERF;
  return TP_ACT_SWIGLU;
}

struct Args {
  std::vector<std::string> pos;
  std::map<std::string, int64_t> opt;
  int64_t i(size_t k) const { return atoll(pos.at(k).c_str()); }
  int64_t o(const char *k, int64_t dflt) const {
    auto it = opt.find(k);
    return it == opt.end() ? dflt : it->second;
  }
};

tp_status run_case(const std::string &op, const Args &a) {
  const int64_t pad = a.o("pad", 0);  // extra elements in every leading dimension
  const bool nows = a.o("nows", 0) != 0;  // pass no workspace (NULL, 0 bytes)
  if (op == "col" || op == "shard" || op == "noalloc" || op == "train") {
    // <dt> <act> T d k i p
    const tp_dtype dt = parse_dt(a.pos[0]);
    const tp_act act = parse_act(a.pos[1]);
    const int64_t T = a.i(2), d = a.i(3), k = a.i(4);
    const int32_t i = (int32_t)a.i(5), p = (int32_t)a.i(6);
    const int64_t es = es_of(dt), s = p > 0 ? k / p : 0;
    const bool sw = act == TP_ACT_SWIGLU, bias = a.o("bias", 0) != 0;
    const int64_t ldx = d + pad, ldw = k + pad, ldy = s + pad, ldz = d + pad;
    void *X = buf(mat(T, d, ldx, es), "X");
    void *W1 = buf(mat(d, k, ldw, es), "W1");
    void *Wu = sw ? buf(mat(d, k, ldw, es), "Wu") : nullptr;
    void *b1 = bias ? buf(k * es, "b1") : nullptr;
    void *Y = buf(mat(T, s, ldy, es), "Y");
    if (op == "col") {
      const size_t wsb = nows ? 0 : tp_workspace_bytes(dt, act, T, d, k, p);
      void *ws = wsb ? buf(wsb, "workspace") : nullptr;
      return tp_col_linear(dt, act, T, d, k, i, p, X, ldx, W1, ldw, Wu, ldw, b1, Y, ldy, ws, wsb,
                           nullptr);
    }
    if (op == "train") {
      const int64_t hw = sw ? 2 * s : s, ldh = hw + pad;
      void *H = buf(mat(T, hw, ldh, es), "H");
      return tp_col_linear_train(dt, act, T, d, k, i, p, X, ldx, W1, ldw, Wu, ldw, b1, Y, ldy, H,
                                 ldh, nullptr);
    }
    void *W2 = buf(mat(k, d, d + pad, es), "W2");
    float *Z = (float *)buf(mat(T, d, ldz, 4), "Z");
    if (op == "noalloc")
      return tp_mlp_shard_noalloc(dt, act, T, d, k, i, p, X, ldx, W1, ldw, Wu, ldw, b1, W2,
                                  d + pad, Y, ldy, Z, ldz, nullptr);
    const size_t wsb = nows ? 0 : tp_workspace_bytes(dt, act, T, d, k, p);
    void *ws = wsb ? buf(wsb, "workspace") : nullptr;
    return tp_mlp_shard(dt, act, T, d, k, i, p, X, ldx, W1, ldw, Wu, ldw, b1, W2, d + pad, Y, ldy,
                        Z, ldz, ws, wsb, nullptr);
  }
  if (op == "row") {  // <dt> T d k i p
    const tp_dtype dt = parse_dt(a.pos[0]);
    const int64_t T = a.i(1), d = a.i(2), k = a.i(3);
    const int32_t i = (int32_t)a.i(4), p = (int32_t)a.i(5);
    const int64_t es = es_of(dt), s = p > 0 ? k / p : 0;
    void *Y = buf(mat(T, s, s + pad, es), "Y");
    void *W2 = buf(mat(k, d, d + pad, es), "W2");
    float *Z = (float *)buf(mat(T, d, d + pad, 4), "Z");
    const size_t wsb = nows ? 0 : tp_workspace_bytes(dt, TP_ACT_NONE, T, d, k, p);
    void *ws = wsb ? buf(wsb, "workspace") : nullptr;
    return tp_row_linear(dt, T, d, k, i, p, Y, s + pad, W2, d + pad, Z, d + pad, ws, wsb, nullptr);
  }
  if (op == "sim") {  // <dt> <act> T d k p
    const tp_dtype dt = parse_dt(a.pos[0]);
    const tp_act act = parse_act(a.pos[1]);
    const int64_t T = a.i(2), d = a.i(3), k = a.i(4);
    const int32_t p = (int32_t)a.i(5);
    const int64_t es = es_of(dt);
    const bool sw = act == TP_ACT_SWIGLU;
    void *X = buf(mat(T, d, d + pad, es), "X");
    void *W1 = buf(mat(d, k, k + pad, es), "W1");
    void *Wu = sw ? buf(mat(d, k, k + pad, es), "Wu") : nullptr;
    void *b1 = a.o("bias", 0) ? buf(k * es, "b1") : nullptr;
    void *W2 = buf(mat(k, d, d + pad, es), "W2");
    float *b2 = a.o("b2", 0) ? (float *)buf(d * 4, "b2") : nullptr;
    void *Y = buf((size_t)(T * k * es), "Y blocks");
    float *Zp = (float *)buf((size_t)(p * T * d * 4), "Z partials");
    float *Z = (float *)buf(mat(T, d, d + pad, 4), "Z");
    const size_t wsb = nows ? 0 : tp_workspace_bytes(dt, act, T, d, k, p);
    void *ws = wsb ? buf(wsb, "workspace") : nullptr;
    return tp_mlp_simulated(dt, act, T, d, k, p, X, d + pad, W1, k + pad, Wu, k + pad, b1, W2,
                            d + pad, b2, Y, Zp, Z, d + pad, ws, wsb, nullptr);
  }
  if (op == "qkv") {  // <dt> T d Hq Hkv dh i p
    const tp_dtype dt = parse_dt(a.pos[0]);
    const int64_t T = a.i(1), d = a.i(2);
    const int32_t Hq = (int32_t)a.i(3), Hkv = (int32_t)a.i(4);
    const int64_t dh = a.i(5);
    const int32_t i = (int32_t)a.i(6), p = (int32_t)a.i(7);
    const int64_t es = es_of(dt), n = (Hq + 2 * (int64_t)Hkv) * dh;
    const int64_t w = p > 0 ? n / p : 0;
    void *X = buf(mat(T, d, d + pad, es), "X");
    void *W = buf(mat(d, n, n + pad, es), "Wqkv");
    void *b = a.o("bias", 0) ? buf(n * es, "bqkv") : nullptr;
    void *O = buf(mat(T, w, w + pad, es), "QKV");
    const size_t wsb = nows ? 0 : tp_qkv_workspace_bytes(dt, T, d, Hq, Hkv, dh, p);
    void *ws = wsb ? buf(wsb, "workspace") : nullptr;
    return tp_qkv_linear(dt, T, d, Hq, Hkv, dh, i, p, X, d + pad, W, n + pad, b, O, w + pad, ws,
                         wsb, nullptr);
  }
  if (op == "attn") {  // nseq S Hq Hkv dh causal
    const int64_t nseq = a.i(0), S = a.i(1);
    const int32_t Hq = (int32_t)a.i(2), Hkv = (int32_t)a.i(3);
    const int64_t dh = a.i(4), T = nseq * S;
    const int32_t causal = (int32_t)a.i(5);
    const int64_t qw = Hq * dh, kw = Hkv * dh;
    void *Q = buf(mat(T, qw, qw + pad, 2), "Q");
    void *K = buf(mat(T, kw, kw + pad, 2), "K");
    void *V = buf(mat(T, kw, kw + pad, 2), "V");
    void *O = buf(mat(T, qw, qw + pad, 2), "O");
    return tp_attention(TP_BF16, nseq, S, Hq, Hkv, dh, causal, Q, qw + pad, K, kw + pad, V,
                        kw + pad, O, qw + pad, nullptr);
  }
  if (op == "bwd") {  // <dt> <act> T d k i p
    const tp_dtype dt = parse_dt(a.pos[0]);
    const tp_act act = parse_act(a.pos[1]);
    const int64_t T = a.i(2), d = a.i(3), k = a.i(4);
    const int32_t i = (int32_t)a.i(5), p = (int32_t)a.i(6);
    const int64_t es = es_of(dt), s = p > 0 ? k / p : 0;
    const bool sw = act == TP_ACT_SWIGLU, db = a.o("db1", 0) != 0;
    const int64_t hw = sw ? 2 * s : s;
    void *X = buf(mat(T, d, d + pad, es), "X");
    void *W1 = buf(mat(d, k, k + pad, es), "W1");
    void *Wu = sw ? buf(mat(d, k, k + pad, es), "Wu") : nullptr;
    void *W2 = buf(mat(k, d, d + pad, es), "W2");
    void *H = buf(mat(T, hw, hw + pad, es), "H");
    void *Y = buf(mat(T, s, s + pad, es), "Y");
    void *dZ = buf(mat(T, d, d + pad, es), "dZ");
    void *dH = buf(mat(T, hw, hw + pad, es), "dH");
    float *dXp = (float *)buf(mat(T, d, d + pad, 4), "dXp");
    float *dW1 = (float *)buf(mat(d, s, s + pad, 4), "dW1");
    float *dWu = sw ? (float *)buf(mat(d, s, s + pad, 4), "dWu") : nullptr;
    float *db1 = db ? (float *)buf(s * 4, "db1") : nullptr;
    float *dW2 = (float *)buf(mat(s, d, d + pad, 4), "dW2");
    const size_t wsb = tp_backward_workspace_bytes(dt, act, T, d, k, p, db ? 1 : 0);
    void *ws = wsb ? buf(wsb, "workspace") : nullptr;
    return tp_mlp_shard_backward(dt, act, T, d, k, i, p, X, d + pad, W1, k + pad, Wu, k + pad, W2,
                                 d + pad, H, hw + pad, Y, s + pad, dZ, d + pad, dH, hw + pad, dXp,
                                 d + pad, dW1, s + pad, dWu, s + pad, db1, dW2, d + pad, ws, wsb,
                                 nullptr);
  }
  if (op == "block") {  // <act> nseq S d Hq Hkv dh k p causal
    const tp_act act = parse_act(a.pos[0]);
    const int64_t nseq = a.i(1), S = a.i(2), d = a.i(3);
    const int32_t Hq = (int32_t)a.i(4), Hkv = (int32_t)a.i(5);
    const int64_t dh = a.i(6), k = a.i(7);
    const int32_t p = (int32_t)a.i(8), causal = (int32_t)a.i(9);
    const int64_t T = nseq * S, n = (Hq + 2 * (int64_t)Hkv) * dh;
    const bool sw = act == TP_ACT_SWIGLU, bias = a.o("bias", 0) != 0;
    float *X = (float *)buf(mat(T, d, d + pad, 4), "X");
    float *g1 = (float *)buf(d * 4, "ln1_g"), *b1n = (float *)buf(d * 4, "ln1_b");
    void *Wqkv = buf(mat(d, n, n + pad, 2), "Wqkv");
    void *bqkv = bias ? buf(n * 2, "bqkv") : nullptr;
    void *WO = buf(mat(Hq * dh, d, d + pad, 2), "WO");
    float *bO = bias ? (float *)buf(d * 4, "bO") : nullptr;
    float *g2 = (float *)buf(d * 4, "ln2_g"), *b2n = (float *)buf(d * 4, "ln2_b");
    void *W1 = buf(mat(d, k, k + pad, 2), "W1");
    void *Wu = sw ? buf(mat(d, k, k + pad, 2), "Wu") : nullptr;
    void *b1 = bias && !sw ? buf(k * 2, "b1") : nullptr;
    void *W2 = buf(mat(k, d, d + pad, 2), "W2");
    float *b2 = bias ? (float *)buf(d * 4, "b2") : nullptr;
    float *Out = a.o("inplace", 0) ? X : (float *)buf(mat(T, d, d + pad, 4), "Out");
    const size_t wsb = tp_block_workspace_bytes(TP_BF16, act, nseq, S, d, Hq, Hkv, dh, k, p);
    void *ws = wsb ? buf(wsb, "workspace") : nullptr;
    return tp_block_simulated(TP_BF16, act, nseq, S, d, Hq, Hkv, dh, k, p, causal, 1e-5f, X,
                              d + pad, g1, b1n, Wqkv, n + pad, bqkv, WO, d + pad, bO, g2, b2n, W1,
                              k + pad, Wu, k + pad, b1, W2, d + pad, b2, Out, d + pad, ws, wsb,
                              nullptr);
  }
  if (op == "psum") {  // T d p
    const int64_t T = a.i(0), d = a.i(1);
    const int32_t p = (int32_t)a.i(2);
    std::vector<const float *> parts;
    for (int j = 0; j < p; ++j) parts.push_back((const float *)buf(mat(T, d, d + pad, 4), "part"));
    float *b2 = a.o("b2", 0) ? (float *)buf(d * 4, "b2") : nullptr;
    float *Z = a.o("inplace", 0) && p > 0 ? (float *)parts[0]
                                          : (float *)buf(mat(T, d, d + pad, 4), "Z");
    return tp_partial_sum(T, d, p, parts.data(), d + pad, b2, Z, d + pad, nullptr);
  }
  if (op == "rln") {  // T d p
    const int64_t T = a.i(0), d = a.i(1);
    const int32_t p = (int32_t)a.i(2);
    std::vector<const float *> parts;
    for (int j = 0; j < p; ++j) parts.push_back((const float *)buf(mat(T, d, d + pad, 4), "part"));
    float *bias = a.o("bias", 0) ? (float *)buf(d * 4, "bias") : nullptr;
    float *R = a.o("R", 1) ? (float *)buf(mat(T, d, d + pad, 4), "R") : nullptr;
    float *X = (float *)buf(mat(T, d, d + pad, 4), "X");
    const bool ln = a.o("ln", 1) != 0;
    float *g = ln ? (float *)buf(d * 4, "gamma") : nullptr;
    float *b = ln ? (float *)buf(d * 4, "beta") : nullptr;
    void *A = ln ? buf(mat(T, d, d + pad, 2), "A") : nullptr;
    return tp_residual_layernorm(T, d, p, parts.data(), d + pad, bias, R, d + pad, X, d + pad, g,
                                 b, 1e-5f, A, d + pad, nullptr);
  }
  fprintf(stderr, "unknown case %s\n", op.c_str());
  exit(2);
}

}  // namespace

int main() {
  std::string line;
  int failed = 0, cases = 0;
  char cbuf[4096];
  while (fgets(cbuf, sizeof cbuf, stdin)) {
    line = cbuf;
    while (!line.empty() && (line.back() == '\n' || line.back() == '\r')) line.pop_back();
    if (line.empty() || line[0] == '#') continue;
    std::istringstream in(line);
    std::string op;
    in >> op;
    const bool expect_error = op == "!";
    if (expect_error) in >> op;
    Args a;
    std::string tok;
    while (in >> tok) {
      const size_t eq = tok.find('=');
      if (eq == std::string::npos)
        a.pos.push_back(tok);
      else
        a.opt[tok.substr(0, eq)] = atoll(tok.c_str() + eq + 1);
    }
    hostcheck::reset();
    g_shrink = (size_t)a.o("shrink", 0);
    const tp_status st = run_case(op, a);
    const hostcheck::Stats &s = hostcheck::stats();
    ++cases;
    bool bad = !s.findings.empty();
    if (expect_error)
      bad |= st == TP_OK || s.launches != 0;
    else
      bad |= st != TP_OK;
    failed += bad;
    printf("CASE %s | status %d launches %ld tiled %ld decode %ld other %ld accesses %ld "
           "findings %zu%s\n",
           line.c_str(), (int)st, s.launches, s.tiled, s.decode, s.checked_other - s.decode,
           s.accesses, s.findings.size(), bad ? " FAILED" : "");
    if (st != TP_OK && !expect_error) printf("ERROR %s\n", tp_last_error_message());
    for (const std::string &f : s.findings) printf("FINDING %s\n", f.c_str());
    if (a.o("kernels", 0))
      for (const std::string &k : s.kernels) printf("KERNEL %s\n", k.c_str());
    fflush(stdout);
  }
  printf("DONE cases %d failed %d\n", cases, failed);
  return failed ? 1 : 0;
}
