"""GPU parity of the shard's backward pass (and of the training forward that
keeps the pre-activation), through the C ABI, against the CPU oracle on the same
seeded inputs.  The oracle recomputes the pre-activation exactly from X and the
weights; the GPU reads it back as the forward stored it (rounded to bf16 like
Y).  Smooth activations are checked on Gaussian data within the bf16 bar; ReLU,
whose derivative is a decision, is checked bit-exactly on integer data where
both sides decide on exact values."""
import numpy as np
import pytest
import torch

import megatron_tensor_mlp_amd as tp
import oracle
from megatron_tensor_mlp_amd import synth
from tests.helpers import assert_bf16_close, assert_f32_close, f64, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def dev(t):
    return None if t is None else t.to(DEV)


def run_train_backward(X, W1, W2, dZ, i, p, act, Wu=None, b1=None, want_db1=False):
    """Training forward of the column step, then the shard backward, on the GPU."""
    T, d = X.shape
    k = W1.shape[1]
    s = k // p
    gated = act == "swiglu"
    hw = 2 * s if gated else s
    dt = X.dtype
    Xd, W1d, W2d, Wud, b1d, dZd = (dev(t) for t in (X, W1, W2, Wu, b1, dZ))
    Y = torch.empty(T, s, dtype=dt, device=DEV)
    H = torch.empty(T, hw, dtype=dt, device=DEV)
    tp.tp_col_linear_train(Xd, W1d, i, p, Y, H, act=act, Wu=Wud, b1=b1d)
    out = {"Y": Y, "H": H,
           "dH": torch.full((T, hw), float("nan"), dtype=dt, device=DEV),
           "dXp": torch.full((T, d), float("nan"), device=DEV),
           "dW1": torch.full((d, s), float("nan"), device=DEV),
           "dW2": torch.full((s, d), float("nan"), device=DEV),
           "dWu": torch.full((d, s), float("nan"), device=DEV) if gated else None,
           "db1": torch.full((s,), float("nan"), device=DEV) if want_db1 else None}
    tp.tp_mlp_shard_backward(Xd, W1d, W2d, H, Y, dZd, i, p, out["dH"], out["dXp"], out["dW1"],
                             out["dW2"], act=act, Wu=Wud, dWu=out["dWu"], db1=out["db1"])
    torch.cuda.synchronize()
    return out


def oracle_bwd(X, W1, W2, dZ, i, p, act, Wu=None, b1=None, want_db1=False):
    return oracle.mlp_shard_backward(f64(X), f64(W1), f64(W2), f64(dZ), i, p, act,
                                     b1=None if b1 is None else f64(b1),
                                     Wu=None if Wu is None else f64(Wu), want_db1=want_db1)


def bf16_case(T, d, k, seed, gated, bias):
    X = synth.gaussian_bf16((T, d), seed)
    W1 = synth.gaussian_bf16((d, k), seed + 1, synth.WEIGHT_STD)
    Wu = synth.gaussian_bf16((d, k), seed + 2, synth.WEIGHT_STD) if gated else None
    b1 = synth.gaussian_bf16((k,), seed + 3, 0.5) if bias else None
    W2 = synth.gaussian_bf16((k, d), seed + 4, synth.WEIGHT_STD)
    dZ = synth.gaussian_bf16((T, d), seed + 5)
    return X, W1, Wu, b1, W2, dZ


# (T, d, k, p, act, bias)
CASES = [
    (300, 264, 1024, 4, "swiglu", False),
    (300, 264, 1024, 4, "gelu_tanh", True),
    (257, 520, 768, 2, "gelu_erf", True),
    (513, 136, 512, 1, "none", False),
    (65, 1032, 2048, 8, "swiglu", False),
    (17, 264, 1024, 4, "gelu_tanh", True),
    (1, 264, 512, 2, "swiglu", False),
    (300, 264, 1056, 4, "swiglu", False),   # k/p = 264: the two dX terms run as two GEMMs
]


@pytest.mark.parametrize("T,d,k,p,act,bias", CASES)
def test_backward_bf16(T, d, k, p, act, bias):
    gated = act == "swiglu"
    X, W1, Wu, b1, W2, dZ = bf16_case(T, d, k, 900 + T, gated, bias)
    for i in sorted({0, p - 1}):
        say(f"backward case T={T} d={d} k={k} p={p} act={act} bias={bias} i={i}")
        g = run_train_backward(X, W1, W2, dZ, i, p, act, Wu=Wu, b1=b1, want_db1=bias)
        r = oracle_bwd(X, W1, W2, dZ, i, p, act, Wu=Wu, b1=b1, want_db1=bias)
        for name in ("dH", "dXp", "dW1", "dW2") + (("dWu",) if gated else ()) + \
                (("db1",) if bias else ()):
            assert_bf16_close(g[name], r[name], name)


def test_train_forward_matches_oracle():
    """Y and the kept pre-activation of the training forward (both bf16 paths'
    shapes; it always runs the tiled kernels)."""
    for T, act, bias in ((300, "gelu_tanh", True), (5, "swiglu", False), (130, "relu", True)):
        gated = act == "swiglu"
        X, W1, Wu, b1, W2, dZ = bf16_case(T, 264, 1024, 40 + T, gated, bias)
        s = 1024 // 4
        Y = torch.empty(T, s, dtype=torch.bfloat16, device=DEV)
        H = torch.empty(T, 2 * s if gated else s, dtype=torch.bfloat16, device=DEV)
        tp.tp_col_linear_train(dev(X), dev(W1), 1, 4, Y, H, act=act, Wu=dev(Wu), b1=dev(b1))
        torch.cuda.synchronize()
        Yr = oracle.col_shard(f64(X), f64(W1), 1, 4, act, b1=None if b1 is None else f64(b1),
                              Wu=None if Wu is None else f64(Wu))
        assert_bf16_close(Y, Yr, "Y")
        Hr = oracle.col_shard(f64(X), f64(W1), 1, 4, "none", b1=None if b1 is None else f64(b1))
        if gated:
            Hr = np.concatenate([Hr, oracle.col_shard(f64(X), f64(Wu), 1, 4, "none")], axis=1)
        assert_bf16_close(H, Hr, "H")


def one_hot_ints(T, d, k, seed):
    """Integer inputs and one-hot +-1 weights: every forward and backward value is
    an exact small integer in bf16 and fp32."""
    rng = np.random.default_rng(seed)
    X = rng.integers(-120, 121, (T, d)).astype(np.float32)
    W1 = np.zeros((d, k), np.float32)
    W2 = np.zeros((k, d), np.float32)
    for g in range(k):
        W1[(7 * g + 3) % d, g] = rng.choice([-1.0, 1.0])
        W2[g, (5 * g + 1) % d] = rng.choice([-1.0, 1.0])
    b1 = rng.integers(-8, 9, (k,)).astype(np.float32)
    dZ = rng.integers(-8, 9, (T, d)).astype(np.float32)
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16)  # noqa: E731
    return bf(X), bf(W1), bf(W2), bf(b1), bf(dZ)


@pytest.mark.parametrize("T", [5, 64, 300])
@pytest.mark.parametrize("act", ["relu", "none"])
def test_backward_bookkeeping_exact(T, act):
    """One-hot integer weights: dH, the dX term, dW1, db1 and dW2 of every shard
    are exact integers, so every transposed-operand index must be right."""
    d, k, p = 264, 1024, 4
    X, W1, W2, b1, dZ = one_hot_ints(T, d, k, T + 7)
    for i in range(p):
        g = run_train_backward(X, W1, W2, dZ, i, p, act, b1=b1, want_db1=True)
        r = oracle_bwd(X, W1, W2, dZ, i, p, act, b1=b1, want_db1=True)
        for name in ("dH", "dXp", "dW1", "dW2", "db1"):
            assert np.array_equal(f64(g[name]), r[name]), f"{name} shard {i}"


def test_backward_f32():
    """fp32 path (Day 41 sizes), every output within 1e-5 of the oracle."""
    X, W1, b1, W2 = synth.tiny_f32_inputs()
    dZ = synth.gaussian_f32((4, 512), 77)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))  # noqa: E731
    for act in ("gelu_tanh", "swiglu"):
        gated = act == "swiglu"
        Wu = synth.gaussian_f32((512, 2048), 78) if gated else None
        bb = None if gated else b1
        for i in (0, 3):
            g = run_train_backward(t(X), t(W1), t(W2), t(dZ), i, 4, act,
                                   Wu=None if Wu is None else t(Wu),
                                   b1=None if bb is None else t(bb), want_db1=not gated)
            r = oracle_bwd(X, W1, W2, dZ, i, 4, act, Wu=Wu, b1=bb, want_db1=not gated)
            for name in ("dH", "dXp", "dW1", "dW2") + (("dWu",) if gated else ("db1",)):
                assert_f32_close(g[name], r[name], f"{act} {name} shard {i}")


def test_backward_dx_terms_sum_to_unsharded():
    """The f operator's backward: the p shards' dX terms, summed on the device,
    equal the unsharded input gradient."""
    T, d, k, p = 200, 264, 1024, 4
    X, W1, Wu, _, W2, dZ = bf16_case(T, d, k, 61, True, False)
    parts = []
    for i in range(p):
        parts.append(run_train_backward(X, W1, W2, dZ, i, p, "swiglu", Wu=Wu)["dXp"])
    dX = torch.empty(T, d, device=DEV)
    tp.tp_partial_sum(parts, dX)
    torch.cuda.synchronize()
    r = oracle_bwd(X, W1, W2, dZ, 0, 1, "swiglu", Wu=Wu)
    assert_bf16_close(dX, r["dXp"], "dX")


def test_backward_zero_tokens_zeroes_weight_gradients():
    d, k, p = 64, 128, 2
    X = torch.empty(0, d, dtype=torch.bfloat16, device=DEV)
    W1 = torch.randn(d, k, device=DEV).to(torch.bfloat16)
    W2 = torch.randn(k, d, device=DEV).to(torch.bfloat16)
    e = torch.empty(0, 64, dtype=torch.bfloat16, device=DEV)
    dW1 = torch.full((d, 64), 5.0, device=DEV)
    dW2 = torch.full((64, d), 5.0, device=DEV)
    db1 = torch.full((64,), 5.0, device=DEV)
    tp.tp_mlp_shard_backward(X, W1, W2, e, e, torch.empty(0, d, dtype=torch.bfloat16, device=DEV),
                             1, p, e, torch.empty(0, d, device=DEV), dW1, dW2, act="gelu_tanh",
                             db1=db1)
    torch.cuda.synchronize()
    assert bool((dW1 == 0).all()) and bool((dW2 == 0).all()) and bool((db1 == 0).all())


# --------------------------------------------------------------------- full size
def test_llama_backward_full_size():
    """Llama-70B SwiGLU shard at TP = 8 (d = 8192, k/p = 3584), T = 4096: dH and
    the dX term on sampled token rows, the weight gradients on sampled columns
    (rows of dW2), each computed by the oracle from the sub-problem it needs."""
    W = synth.WORKLOADS["llama70b_prefill_tp8"]
    Wg, Wu, W2 = synth.llama_shard_weights(W.d, W.s)
    X = synth.llama_tokens(W.T, W.d)
    dZ = synth.gaussian_bf16((W.T, W.d), 46)
    say(f"workload {W.name} backward: T={W.T} d={W.d} s={W.s}")
    g = run_train_backward(X, Wg, W2, dZ, 0, 1, "swiglu", Wu=Wu)
    for name in ("dH", "dXp", "dW1", "dWu", "dW2"):
        assert bool(torch.isfinite(g[name]).all()), name
    rows = [0, 1, 255, 256, 2047, 4095]
    r = oracle_bwd(X[rows], Wg, W2, dZ[rows], 0, 1, "swiglu", Wu=Wu)
    assert_bf16_close(g["dH"][rows], r["dH"], "dH rows")
    assert_bf16_close(g["dXp"][rows], r["dXp"], "dXp rows")
    cols = [0, 1, 127, 128, 1791, 3583]
    rc = oracle_bwd(X, Wg[:, cols], W2[cols, :], dZ, 0, 1, "swiglu", Wu=Wu[:, cols])
    s = W.s
    assert_bf16_close(g["dW1"][:, cols], rc["dW1"], "dWg cols")
    assert_bf16_close(g["dWu"][:, cols], rc["dWu"], "dWu cols")
    assert_bf16_close(g["dW2"][cols, :], rc["dW2"], "dW2 rows")
    gdH = f64(g["dH"])
    assert_bf16_close(np.concatenate([gdH[:, cols], gdH[:, [s + c for c in cols]]], axis=1),
                      rc["dH"], "dH cols")


def test_workspace_shared_with_few_token_forward():
    """The bias gradient's scratch lies past the counter area of the shared
    workspace: a few-token forward after a backward pass that used the same
    (cached) workspace still finds its counters at zero."""
    X, W1, _, b1, W2, dZ = bf16_case(300, 264, 1024, 5, False, True)
    run_train_backward(X, W1, W2, dZ, 1, 4, "gelu_tanh", b1=b1, want_db1=True)
    Xs = X[:3]
    Y = torch.empty(3, 256, dtype=torch.bfloat16, device=DEV)
    Z = torch.empty(3, 264, device=DEV)
    tp.tp_mlp_shard(dev(Xs), dev(W1), dev(W2), 1, 4, Y, Z, act="gelu_tanh", b1=dev(b1))
    torch.cuda.synchronize()
    Yr, Zr = oracle.mlp_shard(f64(Xs), f64(W1), f64(W2), 1, 4, "gelu_tanh", b1=f64(b1))
    assert_bf16_close(Y, Yr, "Y")
    assert_bf16_close(Z, Zr, "Z")
