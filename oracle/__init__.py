"""CPU oracle for one tensor-parallel MLP shard -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain fp64 loops, fp32 instances for the
Day 41 post's printed fp32 check); this module only builds that file with gcc
and marshals numpy arrays to it.  See the header of ``oracle.c`` for what each
function computes and which page passage it follows.

Parity unpinned: nothing here.  Every function is pinned by the CPU tests in
``tests/test_oracle_pins.py`` (printed value, identities, closed forms,
brute force with exact rationals, library routines), the fp32 activations of
the fp32 instances included (against Python's math module in fp64 within the
fp32 evaluation bound, and against torch's fp32 activations).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# The mutation test of the pins (tests/test_oracle_mutants.py) points this at a
# deliberately broken build of oracle.c; nothing else sets it.
_LIB_OVERRIDE = os.environ.get("TPMLP_ORACLE_LIB")

# The oracle's own activation numbering (see oracle.c).
ACT_NONE, ACT_RELU, ACT_GELU_TANH, ACT_GELU_ERF, ACT_SWIGLU = 0, 1, 2, 3, 4
ACT_SILU = ACT_SWIGLU  # scalar helper: kind 4 is SiLU
ACT_BY_NAME = {
    "none": ACT_NONE,
    "relu": ACT_RELU,
    "gelu_tanh": ACT_GELU_TANH,
    "gelu_erf": ACT_GELU_ERF,
    "swiglu": ACT_SWIGLU,
}

_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-std=c11", "-D_DEFAULT_SOURCE", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            build()
            lib = ctypes.CDLL(_LIB)
        i64, i32, ci = ctypes.c_int64, ctypes.c_int32, ctypes.c_int
        vp = ctypes.c_void_p
        lib.oracle_col_shard_f64.argtypes = [i64, i64, i64, i32, i32, vp, vp, vp, vp, ci, vp]
        lib.oracle_row_shard_f64.argtypes = [i64, i64, i64, i32, i32, vp, vp, vp]
        lib.oracle_partial_sum_f64.argtypes = [i64, i64, i32, vp, vp, vp]
        lib.oracle_mlp_unsharded_f64.argtypes = [i64, i64, i64, vp, vp, vp, vp, ci, vp, vp, vp]
        lib.oracle_activation_f64.argtypes = [ci, i64, vp, vp]
        lib.oracle_activation_f64.restype = None
        lib.oracle_linear_f32.argtypes = [i64, i64, i64, vp, vp, vp, ci, vp]
        lib.oracle_col_shard_f32.argtypes = [i64, i64, i64, i32, i32, vp, vp, vp, vp, ci, vp]
        lib.oracle_partial_sum_f32.argtypes = [i64, i64, i32, vp, vp, vp]
        lib.oracle_num_threads.argtypes = []
        lib.oracle_qkv_shard_f64.argtypes = [i64, i64, i32, i32, i64, i32, i32, vp, vp, vp, vp]
        lib.oracle_attention_f64.argtypes = [i64, i64, i32, i32, i64, ci, vp, vp, vp, vp]
        lib.oracle_dactivation_f64.argtypes = [ci, i64, vp, vp]
        lib.oracle_dactivation_f64.restype = None
        lib.oracle_mlp_shard_backward_f64.argtypes = [i64, i64, i64, i32, i32, vp, vp, vp, vp, ci,
                                                      vp, vp, vp, vp, vp, vp, vp, vp]
        cd = ctypes.c_double
        lib.oracle_layernorm_f64.argtypes = [i64, i64, vp, vp, vp, cd, vp]
        lib.oracle_block_f64.argtypes = [i64, i64, i64, i32, i32, i64, i64, ci, ci, cd, vp, vp, vp,
                                         vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, i64, vp,
                                         vp]
        lib.oracle_round_bf16_f64.argtypes = [i64, vp, vp]
        lib.oracle_round_bf16_f64.restype = None
        for name in ("oracle_col_shard_f64", "oracle_row_shard_f64", "oracle_partial_sum_f64",
                     "oracle_mlp_unsharded_f64", "oracle_linear_f32", "oracle_col_shard_f32",
                     "oracle_partial_sum_f32", "oracle_num_threads", "oracle_qkv_shard_f64",
                     "oracle_mlp_shard_backward_f64", "oracle_attention_f64",
                     "oracle_layernorm_f64", "oracle_block_f64"):
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
    return _lib


def _c(a, dtype):
    """Contiguous array of the given dtype (the conversion is exact for bf16/fp32 -> fp64)."""
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _act(act):
    return ACT_BY_NAME[act] if isinstance(act, str) else int(act)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid shard arguments")


def num_threads() -> int:
    return _load().oracle_num_threads()


def col_shard(X, W1, i, p, act, b1=None, Wu=None):
    """Y_i [T, k/p] in fp64 for shard i of p (W1, Wu are the full [d, k] matrices)."""
    lib = _load()
    X, W1, Wu, b1 = _c(X, np.float64), _c(W1, np.float64), _c(Wu, np.float64), _c(b1, np.float64)
    T, d = X.shape
    k = W1.shape[1]
    if k % p:
        raise ValueError("k not divisible by p")
    Y = np.empty((T, k // p), dtype=np.float64)
    _check(lib.oracle_col_shard_f64(T, d, k, i, p, _p(X), _p(W1), _p(Wu), _p(b1), _act(act), _p(Y)),
           "col_shard")
    return Y


def row_shard(Y, W2, i, p):
    """Z_i [T, d] in fp64: shard i's hidden slice times its row block of the full W2 [k, d]."""
    lib = _load()
    Y, W2 = _c(Y, np.float64), _c(W2, np.float64)
    k, d = W2.shape
    T = Y.shape[0]
    if k % p or Y.shape[1] != k // p:
        raise ValueError("shape mismatch")
    Z = np.empty((T, d), dtype=np.float64)
    _check(lib.oracle_row_shard_f64(T, d, k, i, p, _p(Y), _p(W2), _p(Z)), "row_shard")
    return Z


def partial_sum(parts, b2=None):
    """Z = ((parts[0] + parts[1]) + ...) (+ b2), fp64; parts is a sequence of [T, d]."""
    lib = _load()
    P = _c(np.stack([np.asarray(q) for q in parts]), np.float64)
    p, T, d = P.shape
    b2 = _c(b2, np.float64)
    Z = np.empty((T, d), dtype=np.float64)
    _check(lib.oracle_partial_sum_f64(T, d, p, _p(P), _p(b2), _p(Z)), "partial_sum")
    return Z


def mlp_unsharded(X, W1, W2, act, b1=None, Wu=None, b2=None):
    """Z = act(X W1 + b1) W2 + b2 (or SiLU(X Wg) * (X Wu) for swiglu), fp64, computed unsharded."""
    lib = _load()
    X, W1, W2 = _c(X, np.float64), _c(W1, np.float64), _c(W2, np.float64)
    Wu, b1, b2 = _c(Wu, np.float64), _c(b1, np.float64), _c(b2, np.float64)
    T, d = X.shape
    k = W1.shape[1]
    Z = np.empty((T, W2.shape[1]), dtype=np.float64)
    _check(lib.oracle_mlp_unsharded_f64(T, d, k, _p(X), _p(W1), _p(Wu), _p(b1), _act(act),
                                        _p(W2), _p(b2), _p(Z)), "mlp_unsharded")
    return Z


def mlp_shard(X, W1, W2, i, p, act, b1=None, Wu=None):
    """(Y_i, Z_i) for shard i of p, fp64 (column step, then row step)."""
    Y = col_shard(X, W1, i, p, act, b1=b1, Wu=Wu)
    return Y, row_shard(Y, W2, i, p)


def activation(act, x):
    """Element-wise activation in fp64 (kind 'swiglu' / 4 means SiLU here)."""
    lib = _load()
    x = _c(x, np.float64)
    y = np.empty_like(x)
    lib.oracle_activation_f64(_act(act), x.size, _p(x), _p(y))
    return y


def linear_f32(X, W, b=None, act="none"):
    """fp32 unsharded X W + b (then act), summed in fp32 with the index ascending."""
    lib = _load()
    X, W, b = _c(X, np.float32), _c(W, np.float32), _c(b, np.float32)
    T, d = X.shape
    k = W.shape[1]
    Y = np.empty((T, k), dtype=np.float32)
    _check(lib.oracle_linear_f32(T, d, k, _p(X), _p(W), _p(b), _act(act), _p(Y)), "linear_f32")
    return Y


def col_shard_f32(X, W1, i, p, act="none", b1=None, Wu=None):
    """fp32 column step of shard i of p."""
    lib = _load()
    X, W1, Wu, b1 = _c(X, np.float32), _c(W1, np.float32), _c(Wu, np.float32), _c(b1, np.float32)
    T, d = X.shape
    k = W1.shape[1]
    if k % p:
        raise ValueError("k not divisible by p")
    Y = np.empty((T, k // p), dtype=np.float32)
    _check(lib.oracle_col_shard_f32(T, d, k, i, p, _p(X), _p(W1), _p(Wu), _p(b1), _act(act), _p(Y)),
           "col_shard_f32")
    return Y


def partial_sum_f32(parts, b2=None):
    """fp32 Z = ((parts[0] + parts[1]) + ...) (+ b2)."""
    lib = _load()
    P = _c(np.stack([np.asarray(q) for q in parts]), np.float32)
    p, T, d = P.shape
    b2 = _c(b2, np.float32)
    Z = np.empty((T, d), dtype=np.float32)
    _check(lib.oracle_partial_sum_f32(T, d, p, _p(P), _p(b2), _p(Z)), "partial_sum_f32")
    return Z


def qkv_shard(X, Wqkv, Hq, Hkv, dh, i, p, bqkv=None):
    """[Q_i | K_i | V_i] [T, (Hq + 2 Hkv) dh / p] in fp64: the query, key and value
    heads of shard i of p projected from X (Wqkv is the full packed [d, (Hq + 2 Hkv) dh]
    matrix: query heads, then key heads, then value heads)."""
    lib = _load()
    X, W, b = _c(X, np.float64), _c(Wqkv, np.float64), _c(bqkv, np.float64)
    T, d = X.shape
    ncol = (Hq + 2 * Hkv) * dh
    if W.shape != (d, ncol) or Hq % p or Hkv % p:
        raise ValueError("shape mismatch or head counts not divisible by p")
    out = np.empty((T, ncol // p), dtype=np.float64)
    _check(lib.oracle_qkv_shard_f64(T, d, Hq, Hkv, dh, i, p, _p(X), _p(W), _p(b), _p(out)),
           "qkv_shard")
    return out


def dactivation(act, x):
    """Element-wise derivative of the activation in fp64 (kind 'swiglu' / 4 means SiLU')."""
    lib = _load()
    x = _c(x, np.float64)
    y = np.empty_like(x)
    lib.oracle_dactivation_f64(_act(act), x.size, _p(x), _p(y))
    return y


def mlp_shard_backward(X, W1, W2, dZ, i, p, act, b1=None, Wu=None, want_db1=None):
    """Backward pass of shard i of p in fp64, given dZ [T, d].  Returns a dict with
    dH ([T, s]; gated: [T, 2s] = [dG | dU]), dXp [T, d] (this shard's term of dX),
    dW1 [d, s] (gated: dWg), dWu [d, s] (gated only), db1 [s] (when b1 is given and the
    activation is not gated, or want_db1), dW2 [s, d]."""
    lib = _load()
    X, W1, W2, dZ = (_c(a, np.float64) for a in (X, W1, W2, dZ))
    Wu, b1 = _c(Wu, np.float64), _c(b1, np.float64)
    T, d = X.shape
    k = W1.shape[1]
    if k % p:
        raise ValueError("k not divisible by p")
    s = k // p
    gated = _act(act) == ACT_SWIGLU
    if want_db1 is None:
        want_db1 = b1 is not None and not gated
    out = {"dH": np.empty((T, 2 * s if gated else s)), "dXp": np.empty((T, d)),
           "dW1": np.empty((d, s)), "dW2": np.empty((s, d))}
    out["dWu"] = np.empty((d, s)) if gated else None
    out["db1"] = np.empty(s) if want_db1 else None
    _check(lib.oracle_mlp_shard_backward_f64(
        T, d, k, i, p, _p(X), _p(W1), _p(Wu), _p(b1), _act(act), _p(W2), _p(dZ), _p(out["dH"]),
        _p(out["dXp"]), _p(out["dW1"]), _p(out["dWu"]), _p(out["db1"]), _p(out["dW2"])),
        "mlp_shard_backward")
    return out


def attention(Q, K, V, Hq, Hkv, dh, causal=True, S=None):
    """Scaled dot-product attention per head in fp64: Q [T, Hq dh], K and V [T, Hkv dh]
    (query head h reads key/value head h // (Hq / Hkv)); the T tokens are sequences of S
    (default: one sequence of T).  Returns O [T, Hq dh]."""
    lib = _load()
    Q, K, V = _c(Q, np.float64), _c(K, np.float64), _c(V, np.float64)
    T = Q.shape[0]
    S = T if S is None else S
    if Q.shape != (T, Hq * dh) or K.shape != (T, Hkv * dh) or V.shape != (T, Hkv * dh):
        raise ValueError("shape mismatch")
    if S <= 0 and T > 0 or (S > 0 and T % S):
        raise ValueError("T must be a whole number of sequences")
    O = np.empty((T, Hq * dh), dtype=np.float64)
    _check(lib.oracle_attention_f64(T // S if S else 0, S, Hq, Hkv, dh, 1 if causal else 0,
                                    _p(Q), _p(K), _p(V), _p(O)), "attention")
    return O


def layernorm(X, gamma, beta, eps=1e-5):
    """LayerNorm of each row of X [T, d] in fp64 (biased variance, learned scale and
    shift): (x - mean) / sqrt(var + eps) * gamma + beta."""
    lib = _load()
    X = _c(X, np.float64)
    T, d = X.shape
    g, b = _c(gamma, np.float64), _c(beta, np.float64)
    if g.shape != (d,) or b.shape != (d,):
        raise ValueError("shape mismatch")
    Y = np.empty((T, d), dtype=np.float64)
    _check(lib.oracle_layernorm_f64(T, d, _p(X), _p(g), _p(b), float(eps), _p(Y)), "layernorm")
    return Y


def block(X, Hq, Hkv, dh, act, ln1, Wqkv, WO, ln2, W1, W2, S=None, causal=True, eps=1e-5,
          bqkv=None, bO=None, Wu=None, b1=None, b2=None, rows=None, mirror=False):
    """One pre-LayerNorm transformer block in fp64, unsharded: X [T, d] (sequences of
    S tokens, default one of T); ln1 and ln2 are (gamma, beta) pairs; Wqkv [d, (Hq +
    2 Hkv) dh], WO [Hq dh, d], W1 (and Wu) [d, k], W2 [k, d].  Returns the block output
    for the token rows listed in `rows` (default all), [len(rows), d].  mirror=True is
    a diagnostic: the activations a bf16 implementation stores (the LayerNorm outputs,
    QKV, the attention output, the FFN hidden activation) are rounded to bf16."""
    lib = _load()
    X = _c(X, np.float64)
    T, d = X.shape
    S = T if S is None else S
    if S <= 0 and T > 0 or (S > 0 and T % S):
        raise ValueError("T must be a whole number of sequences")
    k = W1.shape[1]
    f = lambda a: _c(a, np.float64)  # noqa: E731
    args = [f(ln1[0]), f(ln1[1]), f(Wqkv), f(bqkv), f(WO), f(bO), f(ln2[0]), f(ln2[1]), f(W1),
            f(Wu), f(b1), f(W2), f(b2)]
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n = T if r is None else len(r)
    Out = np.empty((n, d), dtype=np.float64)
    _check(lib.oracle_block_f64(T // S if S else 0, S, d, Hq, Hkv, dh, k, 1 if causal else 0,
                                _act(act), float(eps), _p(X), *[_p(a) for a in args],
                                1 if mirror else 0, n, _p(r), _p(Out)), "block")
    return Out


def round_bf16(x):
    """x rounded to fp32, then to the nearest bf16 (ties to even), as fp64."""
    lib = _load()
    x = _c(x, np.float64)
    y = np.empty_like(x)
    lib.oracle_round_bf16_f64(x.size, _p(x), _p(y))
    return y


def block_storage_error(X, Hq, Hkv, dh, act, ln1, Wqkv, WO, ln2, W1, W2, S=None, causal=True,
                        eps=1e-5, bqkv=None, bO=None, Wu=None, b1=None, b2=None, rows=None,
                        rel=2.0 ** -8, draws=2, seed=0):
    """An a-priori estimate of the error that storing a block's activations in bf16
    causes in the block's update (output minus input), computed from the exact
    oracle's own activations.

    The block is composed from this module's functions exactly as ``block`` computes
    it (LayerNorm, the full QKV projection, attention, the output projection plus its
    bias and the residual, LayerNorm, the FFN, its bias and the residual), once as is
    and ``draws`` more times with every activation a bf16 implementation stores -- the
    two LayerNorm outputs, Q, K, V, the attention output and the FFN hidden activation
    -- multiplied element-wise by (1 + rel * xi), xi independent and uniform on
    [-1, 1] (numpy default_rng(seed + draw)).  rel = 2^-8 is bf16's unit roundoff,
    the largest relative error a round to nearest bf16 makes; this is a model of the
    size of that error, not the rounding itself.

    Returns (U, e_fro, e_max): the exact update for the token rows listed in ``rows``
    (default all), and the root mean square over the draws of the perturbed updates'
    relative Frobenius distance ||dU|| / ||U|| and relative largest distance
    max|dU| / max|U| from it."""
    X = _c(X, np.float64)
    T, d = X.shape
    S = T if S is None else S
    r = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    f = lambda a: None if a is None else _c(a, np.float64)  # noqa: E731
    Wqkv, WO, W1, W2, Wu = f(Wqkv), f(WO), f(W1), f(W2), f(Wu)
    bqkv, bO, b1, b2 = f(bqkv), f(bO), f(b1), f(b2)
    qw, kw = Hq * dh, Hkv * dh

    def run(pert):
        A1 = pert(layernorm(X, ln1[0], ln1[1], eps))
        QKV = qkv_shard(A1, Wqkv, Hq, Hkv, dh, 0, 1, bqkv=bqkv)
        Q, K, V = (pert(np.ascontiguousarray(QKV[:, a:b]))
                   for a, b in ((0, qw), (qw, qw + kw), (qw + kw, qw + 2 * kw)))
        O = pert(attention(Q, K, V, Hq, Hkv, dh, causal=causal, S=S))
        P = row_shard(O[r], WO, 0, 1)
        X1 = X[r] + (P + bO if bO is not None else P)
        A2 = pert(layernorm(X1, ln2[0], ln2[1], eps))
        Y = pert(col_shard(A2, W1, 0, 1, act, b1=b1, Wu=Wu))
        Z = row_shard(Y, W2, 0, 1)
        if b2 is not None:
            Z = Z + b2
        return (X1 + Z) - X[r]

    U = run(lambda a: a)
    nu, mu = float(np.linalg.norm(U)), float(np.max(np.abs(U))) if U.size else 0.0
    e_fro = e_max = 0.0
    for q in range(draws):
        rng = np.random.default_rng(seed + q)
        dU = run(lambda a: a * (1.0 + rel * rng.uniform(-1.0, 1.0, a.shape))) - U
        e_fro += (float(np.linalg.norm(dU)) / max(nu, 1e-300)) ** 2
        e_max += (float(np.max(np.abs(dU))) / max(mu, 1e-300) if dU.size else 0.0) ** 2
    return U, (e_fro / max(draws, 1)) ** 0.5, (e_max / max(draws, 1)) ** 0.5
