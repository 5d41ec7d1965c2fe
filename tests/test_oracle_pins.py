"""Pins of the CPU oracle to what the pages and the mathematics fix.

None of these tests re-types the oracle's formulas: each compares it with a
value the pages print, an identity, a closed form, a special case, brute force
with exact rationals, or an independent library routine.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from megatron_tensor_mlp_amd import synth


def rel_fro(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# ---------------------------------------------------------------- P-1 --------
def test_day41_printed_concat_error_fp32(golden):
    """Day 41 post, 'Simulating column parallel linear': concatenating the column
    shards reproduces x @ W + b with a printed max error of 0.00e+00 (fp32)."""
    g = golden("day41_column_concat.txt")
    assert g["dtype"] == "float32"
    rs = np.random.RandomState(int(g["seed"]))
    T, d, k, p = (int(g[n]) for n in ("batch", "in_features", "out_features", "num_gpus"))
    x = rs.randn(T, d).astype(np.float32)
    W = rs.randn(d, k).astype(np.float32)
    b = rs.randn(k).astype(np.float32)
    full = oracle.linear_f32(x, W, b)
    shards = [oracle.col_shard_f32(x, W, i, p, "none", b1=b) for i in range(p)]
    concat = np.concatenate(shards, axis=1)
    assert concat.shape == full.shape == (T, k)
    max_err = float(np.max(np.abs(full - concat)))
    assert max_err == float(g["max_error"]) == 0.0
    # the same holds after a local element-wise activation
    for act in ("gelu_tanh", "gelu_erf", "relu"):
        full_a = oracle.linear_f32(x, W, b, act)
        cat_a = np.concatenate([oracle.col_shard_f32(x, W, i, p, act, b1=b) for i in range(p)], 1)
        assert np.array_equal(full_a, cat_a)
    # and the fp32 result is a genuine fp32 matmul (not something else that is
    # trivially equal): it agrees with fp64 numpy to fp32 rounding
    ref = x.astype(np.float64) @ W.astype(np.float64) + b
    assert rel_fro(full, ref) < 1e-6


def test_tiny_workload_generator_matches_day41_draw():
    """The tiny fp32 workload draws x, W, b exactly as the Day 41 post does."""
    X, W1, b1, W2 = synth.tiny_f32_inputs()
    rs = np.random.RandomState(42)
    assert np.array_equal(X, rs.randn(4, 512).astype(np.float32))
    assert np.array_equal(W1, rs.randn(512, 2048).astype(np.float32))
    assert np.array_equal(b1, rs.randn(2048).astype(np.float32))
    assert W2.shape == (2048, 512) and W2.dtype == np.float32
    assert 0.8 / math.sqrt(2048) < W2.std() < 1.2 / math.sqrt(2048)


def test_fp64_concat_bit_exact_all_acts():
    """Column concat equals the unsharded column step bit-for-bit in fp64 too."""
    X, W1, b1, W2 = synth.tiny_f32_inputs()
    for act in ("none", "relu", "gelu_tanh", "gelu_erf"):
        full = oracle.col_shard(X, W1, 0, 1, act, b1=b1)
        cat = np.concatenate([oracle.col_shard(X, W1, i, 4, act, b1=b1) for i in range(4)], 1)
        assert np.array_equal(full, cat), act
    Wu = synth.gaussian_f32((512, 2048), 7)
    full = oracle.col_shard(X, W1, 0, 1, "swiglu", Wu=Wu)
    cat = np.concatenate([oracle.col_shard(X, W1, i, 4, "swiglu", Wu=Wu) for i in range(4)], 1)
    assert np.array_equal(full, cat)


# ---------------------------------------------------------------- P-2 --------
@pytest.mark.parametrize("act", ["gelu_tanh", "gelu_erf", "relu", "swiglu"])
@pytest.mark.parametrize("p", [1, 2, 4, 8])
def test_sum_of_row_partials_equals_unsharded(act, p):
    """'Transformer math: tensor parallel', row-parallel and MLP sections: the p
    partial outputs sum to the unsharded MLP output (up to reassociation)."""
    T, d, k = 5, 24, 64
    X, W1, Wu, b1, W2 = (None if a is None else a.to(torch.float64).numpy()
                         for a in synth.small_case(T, d, k, 11, act == "swiglu",
                                                   act != "swiglu", w_std=0.3))
    b2 = synth.gaussian_f32((d,), 99).astype(np.float64)
    parts = [oracle.mlp_shard(X, W1, W2, i, p, act, b1=b1, Wu=Wu)[1] for i in range(p)]
    Z = oracle.partial_sum(parts, b2)
    Zfull = oracle.mlp_unsharded(X, W1, W2, act, b1=b1, Wu=Wu, b2=b2)
    assert rel_fro(Z, Zfull) <= 1e-12


# ---------------------------------------------------------------- P-3 --------
@pytest.mark.parametrize("p", [1, 3, 4])
def test_linear_closed_form(p):
    """'Tensor Parallelism Explained', section 1.B: with no activation the
    reduced result is X (W W'), a closed form computed here with numpy."""
    rng = np.random.default_rng(5)
    T, d, k = 6, 20, 36
    X = rng.standard_normal((T, d))
    W1 = rng.standard_normal((d, k))
    W2 = rng.standard_normal((k, d))
    parts = [oracle.mlp_shard(X, W1, W2, i, p, "none")[1] for i in range(p)]
    closed = X @ (W1 @ W2)
    assert rel_fro(oracle.partial_sum(parts), closed) <= 1e-12
    assert rel_fro(oracle.mlp_unsharded(X, W1, W2, "none"), closed) <= 1e-12


# ---------------------------------------------------------------- P-4 --------
@pytest.mark.parametrize("act", ["gelu_tanh", "relu", "swiglu", "gelu_erf"])
def test_p1_is_bit_identical_to_unsharded(act):
    """'Building GPT from Scratch, Part 9', section 'Running This On Your
    MacBook?': TP=1 is the original model.  One shard of one is bit-identical."""
    X, W1, Wu, b1, W2 = (None if a is None else a.to(torch.float64).numpy()
                         for a in synth.small_case(7, 40, 48, 3, act == "swiglu", act != "swiglu"))
    b2 = np.linspace(-1, 1, 40)
    Y, Zi = oracle.mlp_shard(X, W1, W2, 0, 1, act, b1=b1, Wu=Wu)
    Z = oracle.partial_sum([Zi], b2)
    assert np.array_equal(Z, oracle.mlp_unsharded(X, W1, W2, act, b1=b1, Wu=Wu, b2=b2))


# ---------------------------------------------------------------- P-5 --------
def test_negative_control_activation_on_partial_sums():
    """'Transformer math: tensor parallel', MLP section: putting the nonlinearity
    on partial sums (splitting the first weight by rows) is wrong, while with no
    nonlinearity the two orders agree.  The oracle must show both."""
    rng = np.random.default_rng(1)
    T, d, k = 8, 32, 16
    X = rng.standard_normal((T, d))
    W = rng.standard_normal((d, k)) / math.sqrt(d)
    h = d // 2
    for act, should_match in (("none", True), ("gelu_tanh", False), ("gelu_erf", False)):
        right = oracle.col_shard(X, W, 0, 1, act)
        wrong = (oracle.col_shard(X[:, :h], W[:h], 0, 1, act)
                 + oracle.col_shard(X[:, h:], W[h:], 0, 1, act))
        err = rel_fro(wrong, right)
        if should_match:
            assert err <= 1e-12
        else:
            assert err > 0.1, (act, err)


# ---------------------------------------------------------------- P-6 --------
def _brute_force(X, W1, b1, W2, b2, p, relu):
    """Exact rational evaluation of the sharded MLP straight from the block
    formulas: Y_i = act(X A_i + b_i), Z = sum_i Y_i B_i + b2."""
    T, d = len(X), len(X[0])
    k = len(W1[0])
    s = k // p
    Z = [[Fraction(0)] * len(W2[0]) for _ in range(T)]
    for i in range(p):
        for t in range(T):
            y = []
            for j in range(s):
                v = sum((Fraction(X[t][c]) * Fraction(W1[c][i * s + j]) for c in range(d)),
                        Fraction(0)) + Fraction(b1[i * s + j])
                y.append(max(v, Fraction(0)) if relu else v)
            for n in range(len(W2[0])):
                Z[t][n] += sum((y[j] * Fraction(W2[i * s + j][n]) for j in range(s)), Fraction(0))
    return [[Z[t][n] + Fraction(b2[n]) for n in range(len(W2[0]))] for t in range(T)]


@pytest.mark.parametrize("T,d,s,p", [(1, 1, 1, 1), (2, 3, 1, 4), (3, 5, 3, 2), (3, 4, 2, 3),
                                     (2, 5, 3, 4), (1, 2, 3, 1)])
@pytest.mark.parametrize("relu", [False, True])
def test_brute_force_exact_rationals(T, d, s, p, relu):
    """Brute force on tiny shapes with small integers: the oracle is exact."""
    rng = np.random.default_rng(T * 100 + d * 10 + s + p)
    k = s * p
    X = rng.integers(-4, 5, (T, d)).astype(np.float64)
    W1 = rng.integers(-3, 4, (d, k)).astype(np.float64)
    b1 = rng.integers(-5, 6, (k,)).astype(np.float64)
    W2 = rng.integers(-3, 4, (k, d)).astype(np.float64)
    b2 = rng.integers(-5, 6, (d,)).astype(np.float64)
    act = "relu" if relu else "none"
    expect = _brute_force(X.tolist(), W1.tolist(), b1.tolist(), W2.tolist(), b2.tolist(), p, relu)
    parts = [oracle.mlp_shard(X, W1, W2, i, p, act, b1=b1)[1] for i in range(p)]
    got = oracle.partial_sum(parts, b2)
    assert [[Fraction(v) for v in row] for row in got.tolist()] == expect
    got_u = oracle.mlp_unsharded(X, W1, W2, act, b1=b1, b2=b2)
    assert [[Fraction(v) for v in row] for row in got_u.tolist()] == expect


def test_brute_force_swiglu_small():
    """SwiGLU ('Tensor Parallelism Explained', section 2.B): Swish(X Wg_i) times
    (X Wu_i), evaluated here term by term with Python's math.exp."""
    rng = np.random.default_rng(8)
    T, d, k, p = 2, 3, 4, 2
    X = rng.integers(-3, 4, (T, d)).astype(np.float64)
    Wg = rng.integers(-2, 3, (d, k)).astype(np.float64)
    Wu = rng.integers(-2, 3, (d, k)).astype(np.float64)
    W2 = rng.integers(-2, 3, (k, d)).astype(np.float64)
    s = k // p
    for i in range(p):
        Y, Zi = oracle.mlp_shard(X, Wg, W2, i, p, "swiglu", Wu=Wu)
        for t in range(T):
            for j in range(s):
                g = sum(X[t][c] * Wg[c][i * s + j] for c in range(d))
                u = sum(X[t][c] * Wu[c][i * s + j] for c in range(d))
                assert Y[t][j] == pytest.approx(g / (1 + math.exp(-g)) * u, rel=1e-14, abs=1e-14)


# ---------------------------------------------------------------- P-7 --------
def test_matmul_against_numpy():
    rng = np.random.default_rng(2)
    T, d, k, p = 9, 70, 96, 4
    X = rng.standard_normal((T, d))
    W1 = rng.standard_normal((d, k))
    W2 = rng.standard_normal((k, d))
    s = k // p
    for i in range(p):
        Y = oracle.col_shard(X, W1, i, p, "none")
        assert rel_fro(Y, X @ W1[:, i * s:(i + 1) * s]) <= 1e-13
        Z = oracle.row_shard(Y, W2, i, p)
        assert rel_fro(Z, Y @ W2[i * s:(i + 1) * s, :]) <= 1e-13


GRID = np.array([0.0, 1e-8, -1e-8, 1.0, -1.0, 3.0, -3.0, 10.0, -10.0, 30.0, -30.0, 0.5, -0.5,
                 2.25, -7.75, 1e-3, -1e-3])


def test_activations_against_library_routines():
    x = np.concatenate([GRID, np.linspace(-12, 12, 1001)])
    xt = torch.from_numpy(x)
    ref_tanh = torch.nn.functional.gelu(xt, approximate="tanh").numpy()
    ref_erf = torch.nn.functional.gelu(xt, approximate="none").numpy()
    ref_silu = torch.nn.functional.silu(xt).numpy()
    np.testing.assert_allclose(oracle.activation("gelu_tanh", x), ref_tanh, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(oracle.activation("gelu_erf", x), ref_erf, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(oracle.activation("swiglu", x), ref_silu, rtol=1e-13, atol=1e-15)
    assert np.array_equal(oracle.activation("relu", x), np.maximum(x, 0.0))
    assert np.array_equal(oracle.activation("none", x), x)
    # scalar spot checks against Python's math module
    for v in GRID:
        assert oracle.activation("gelu_erf", np.array([v]))[0] == pytest.approx(
            0.5 * v * math.erfc(-v / math.sqrt(2)), rel=1e-13, abs=1e-15)
        assert oracle.activation("swiglu", np.array([v]))[0] == pytest.approx(
            v * 0.5 * (1 + math.tanh(v / 2)), rel=1e-13, abs=1e-15)


F32_GRID = np.concatenate([GRID, np.linspace(-40.0, 40.0, 641), [-88.5, -90.0, -100.0, 88.0]])


def _math_gelu_tanh(v):
    c = math.sqrt(2.0 / math.pi)
    return 0.5 * v * (1.0 + math.tanh(c * (v + 0.044715 * v ** 3)))


def _math_silu(v):
    # x * sigmoid(x) through the identity sigmoid(x) = (1 + tanh(x/2)) / 2
    return v * 0.5 * (1.0 + math.tanh(v / 2.0))


@pytest.mark.parametrize("act", ["gelu_tanh", "gelu_erf", "swiglu"])
def test_fp32_activations_against_fp64_library(act):
    """The fp32 path's activations (Day 41 post, 'Simulating column parallel
    linear', in fp32) against Python's math module in fp64 at the same fp32
    inputs.  The bound is a few fp32 ulps of |y| + |x|: the GeLU forms compute
    0.5 x (1 + F) with F near -1 for negative x, so their fp32 evaluation can
    lose all of its relative accuracy but never more than ulp(1) in the factor
    (1 + F); an absolute floor of 1e-30 covers SiLU's tail, where the true value
    underflows fp32.  A dropped term or a flipped sign misses by orders of
    magnitude more (checked by planted mistakes).  The inputs reach
    the activation exactly: X = [[1]] and W = the grid, so X W + b = the grid in
    fp32 with no rounding.  Both fp32 entry points (unsharded and one shard of 4)
    are checked; the gated variant's up factor is 1."""
    h = F32_GRID.astype(np.float32)
    n = h.size - (h.size % 4)
    h = h[:n]
    X = np.ones((1, 1), np.float32)
    W = h.reshape(1, n)
    if act == "gelu_tanh":
        ref = np.array([_math_gelu_tanh(float(v)) for v in h])
    elif act == "gelu_erf":
        ref = np.array([0.5 * float(v) * math.erfc(-float(v) / math.sqrt(2.0)) for v in h])
    else:
        ref = np.array([_math_silu(float(v)) for v in h])
    if act == "swiglu":  # the unsharded fp32 linear has no gated form: one shard of one
        ones = np.ones_like(W)
        got_full = oracle.col_shard_f32(X, W, 0, 1, act, Wu=ones)[0].astype(np.float64)
        shards = [oracle.col_shard_f32(X, W, i, 4, act, Wu=ones) for i in range(4)]
    else:
        got_full = oracle.linear_f32(X, W, None, act)[0].astype(np.float64)
        shards = [oracle.col_shard_f32(X, W, i, 4, act) for i in range(4)]
    got_shard = np.concatenate(shards, axis=1)[0].astype(np.float64)
    tol = 8 * 2.0 ** -24 * (np.abs(ref) + np.abs(h.astype(np.float64))) + 1e-30
    for got in (got_full, got_shard):
        bad = np.abs(got - ref) > tol
        assert not bad.any(), (act, h[bad][:5], got[bad][:5], ref[bad][:5])
    # torch's fp32 activations agree too (an independent fp32 implementation)
    ht = torch.from_numpy(h)
    tref = {"gelu_tanh": lambda t: torch.nn.functional.gelu(t, approximate="tanh"),
            "gelu_erf": lambda t: torch.nn.functional.gelu(t, approximate="none"),
            "swiglu": torch.nn.functional.silu}[act](ht).double().numpy()
    assert np.all(np.abs(got_full - tref) <= 2 * tol)


def test_activation_odd_part_identities():
    """act(x) - act(-x) = x for both GeLU forms and SiLU (each is x times a
    function F with F(x) + F(-x) = 1); GeLU(0) = SiLU(0) = 0; large |x| limits."""
    x = np.linspace(-9, 9, 721)
    for act in ("gelu_tanh", "gelu_erf", "swiglu"):
        y, ym = oracle.activation(act, x), oracle.activation(act, -x)
        np.testing.assert_allclose(y - ym, x, rtol=1e-13, atol=1e-14)
        assert oracle.activation(act, np.array([0.0]))[0] == 0.0
        big = oracle.activation(act, np.array([40.0, -40.0]))
        assert big[0] == pytest.approx(40.0, rel=1e-12) and abs(big[1]) < 1e-12


# ---------------------------------------------------------------- P-8 --------
def one_hot_case(T, d, k, seed):
    """Integer one-hot weights: W1 column g has a single +-1 at row (7g+3) mod d,
    W2 row g has a single +-1 at column (5g+1) mod d; X small integers."""
    rng = np.random.default_rng(seed)
    X = rng.integers(-256, 257, (T, d)).astype(np.float64)
    W1 = np.zeros((d, k))
    W2 = np.zeros((k, d))
    sg1 = rng.choice([-1.0, 1.0], k)
    sg2 = rng.choice([-1.0, 1.0], k)
    for g in range(k):
        W1[(7 * g + 3) % d, g] = sg1[g]
        W2[g, (5 * g + 1) % d] = sg2[g]
    b1 = rng.integers(-8, 9, (k,)).astype(np.float64)
    return X, W1, W2, b1, sg1, sg2


@pytest.mark.parametrize("p", [1, 2, 4, 8])
def test_bookkeeping_one_hot(p):
    """Day 41 post: shard i owns columns [i*s, (i+1)*s) of the first weight and
    the same rows of the second.  With one-hot integer weights every output is a
    known integer, so an off-by-shard or transposed index fails exactly."""
    T, d, k = 5, 24, 64
    X, W1, W2, b1, sg1, sg2 = one_hot_case(T, d, k, p)
    s = k // p
    for i in range(p):
        Y, Zi = oracle.mlp_shard(X, W1, W2, i, p, "relu", b1=b1)
        expY = np.zeros((T, s))
        for j in range(s):
            g = i * s + j
            expY[:, j] = np.maximum(sg1[g] * X[:, (7 * g + 3) % d] + b1[g], 0)
        assert np.array_equal(Y, expY)
        expZ = np.zeros((T, d))
        for j in range(s):
            g = i * s + j
            expZ[:, (5 * g + 1) % d] += sg2[g] * expY[:, j]
        assert np.array_equal(Zi, expZ)


def test_shard_rule_errors():
    """The shard rule: k must be divisible by p, 0 <= i < p ('Tensor Parallelism
    Explained', section 4: a non-dividing degree fails at startup)."""
    X = np.zeros((2, 4))
    W = np.zeros((4, 10))
    with pytest.raises(ValueError):
        oracle.col_shard(X, W, 0, 4, "none")
    with pytest.raises(ValueError):
        oracle.col_shard(X, W, 2, 2, "none")
    with pytest.raises(ValueError):
        oracle.col_shard(X, W, -1, 2, "none")


def test_llama_shard_width(golden):
    """'What is Tensor Parallelism?', Llama 3.1 70B worked example: 28672 / 8 = 3584
    feed-forward columns per GPU; the oracle's shard of a [d, 28672] weight has
    that many columns and its partial has the full [T, 8192] shape."""
    g = golden("llama70b_tp8_shapes.txt")
    k, p, s = int(g["ffn_size"]), int(g["tp"]), int(g["ffn_columns_per_gpu"])
    d = 8
    X = np.ones((1, d))
    W1 = np.zeros((d, k))
    Y = oracle.col_shard(X, W1, p - 1, p, "none")
    assert Y.shape == (1, s)
    hidden = int(g["hidden_size"])
    W2 = np.zeros((k, hidden))
    Z = oracle.row_shard(Y, W2, p - 1, p)
    assert Z.shape == (1, hidden)
    tokens = int(g["prompt_tokens"])
    assert tokens * hidden * 2 == pytest.approx(float(g["allreduce_tensor_bytes_bf16"]), rel=1e-3)
    assert hidden * 2 == pytest.approx(float(g["decode_tensor_bytes_bf16"]), rel=0.05)


def test_gpt_ffn_shard_shapes(golden):
    """'Transformer math: tensor parallel', worked example: four [4096, 4096]
    column shards of a [4096, 16384] weight; a [4096, 4096] partial of 33.5 MB."""
    g = golden("gpt_ffn_p4_shapes.txt")
    d, dff, p = int(g["d"]), int(g["d_ff"]), int(g["p"])
    assert (d, dff // p) == (int(g["column_shard_rows"]), int(g["column_shard_cols"]))
    assert (dff // p, d) == (int(g["row_shard_rows"]), int(g["row_shard_cols"]))
    assert int(g["tokens"]) * d * 2 == pytest.approx(float(g["partial_bytes_16bit"]), rel=2e-3)
    # the oracle's shards of a (narrow) [8, 16384] weight have 4096 columns
    Y = oracle.col_shard(np.ones((1, 8)), np.zeros((8, dff)), 3, p, "none")
    assert Y.shape == (1, dff // p)


# ---------------------------------------------------------------- P-9 --------
def test_bf16_inputs_round_trip_exactly():
    """Inputs are rounded to bf16 once (RNE); widening them to fp64 for the
    oracle is exact, and the RNE ties go to even."""
    a = synth.gaussian_bf16((1000,), 3)
    assert torch.equal(a.to(torch.float64).to(torch.bfloat16), a)
    ties = torch.tensor([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8)],
                        dtype=torch.float32).to(torch.bfloat16).to(torch.float64)
    assert ties.tolist() == [1.0, 1.0 + 2.0 ** -6, -1.0]


def test_partial_sum_order_fp32():
    """fp32 reduction adds shard 0 first, then 1, ...; the order is observable."""
    parts = [np.array([[1e8]], np.float32), np.array([[1.0]], np.float32),
             np.array([[-1e8]], np.float32)]
    assert oracle.partial_sum_f32(parts)[0, 0] == np.float32(0.0)  # (1e8 + 1) - 1e8 in fp32
    parts2 = [parts[0], parts[2], parts[1]]
    assert oracle.partial_sum_f32(parts2)[0, 0] == np.float32(1.0)
    b2 = np.array([0.5], np.float32)
    assert oracle.partial_sum_f32(parts2, b2)[0, 0] == np.float32(1.5)


# ---------------------------------------------------------------- P-10 -------
# The attention projections: QKV column-parallel by heads, W_O row-parallel.
def _int_case(T, d, ncol, seed):
    """Small-integer inputs: every fp64 product and sum below is exact."""
    rng = np.random.default_rng(seed)
    X = rng.integers(-4, 5, (T, d)).astype(np.float64)
    W = rng.integers(-4, 5, (d, ncol)).astype(np.float64)
    b = rng.integers(-9, 10, (ncol,)).astype(np.float64)
    return X, W, b


@pytest.mark.parametrize("Hq,Hkv,dh,p", [(4, 4, 3, 1), (4, 4, 3, 2), (8, 2, 2, 2), (8, 4, 5, 4),
                                         (6, 3, 1, 3)])
def test_qkv_shards_reassemble_full_projection(Hq, Hkv, dh, p):
    """Each GPU's Q, K and V columns are exactly its heads' columns of the full
    projection X Wqkv + b: putting the shards' query heads side by side in shard
    order gives the full query block, and the same for keys and values
    ('Transformer math: tensor parallel', section "Attention: parallel across
    heads").  Integer inputs make the comparison with numpy's matmul exact."""
    T, d = 5, 7
    ncol = (Hq + 2 * Hkv) * dh
    X, W, b = _int_case(T, d, ncol, Hq * 100 + p)
    full = X @ W + b
    qw, kw = Hq * dh // p, Hkv * dh // p
    shards = [oracle.qkv_shard(X, W, Hq, Hkv, dh, i, p, bqkv=b) for i in range(p)]
    for s in shards:
        assert s.shape == (T, qw + 2 * kw)
    Q = np.concatenate([s[:, :qw] for s in shards], axis=1)
    K = np.concatenate([s[:, qw:qw + kw] for s in shards], axis=1)
    V = np.concatenate([s[:, qw + kw:] for s in shards], axis=1)
    assert np.array_equal(Q, full[:, :Hq * dh])
    assert np.array_equal(K, full[:, Hq * dh:(Hq + Hkv) * dh])
    assert np.array_equal(V, full[:, (Hq + Hkv) * dh:])
    # without a bias: the same columns of X Wqkv
    s0 = oracle.qkv_shard(X, W, Hq, Hkv, dh, p - 1, p)
    assert np.array_equal(s0, shards[p - 1] - np.concatenate(
        [b[(p - 1) * qw:p * qw], b[Hq * dh + (p - 1) * kw:Hq * dh + p * kw],
         b[(Hq + Hkv) * dh + (p - 1) * kw:(Hq + Hkv) * dh + p * kw]]))


def _softmax_attention(Q, K, V):
    """softmax(Q K^T / sqrt(dk)) V for one head, fp64 (scaled dot-product attention)."""
    s = Q @ K.T / math.sqrt(Q.shape[1])
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    return (e / e.sum(axis=1, keepdims=True)) @ V


def _heads_attention(Q, K, V, hq, hkv, dh):
    """Per-head attention over [T, hq dh] queries and [T, hkv dh] keys/values;
    query head h reads key/value head h // (hq / hkv) (grouped heads)."""
    g = hq // hkv
    outs = []
    for h in range(hq):
        c = h // g
        outs.append(_softmax_attention(Q[:, h * dh:(h + 1) * dh], K[:, c * dh:(c + 1) * dh],
                                       V[:, c * dh:(c + 1) * dh]))
    return np.concatenate(outs, axis=1)


@pytest.mark.parametrize("Hq,Hkv,dh,p", [(4, 4, 4, 2), (8, 2, 4, 2), (8, 4, 2, 4), (4, 1, 4, 1)])
def test_head_split_attention_sums_to_full(Hq, Hkv, dh, p):
    """Multi-head attention is the concatenation of the heads times W_O, i.e. a
    sum over heads of head_h times W_O's rows of head h ('Building GPT from
    Scratch, Part 9', section "Why This Works").  So per-shard attention on the
    shard's Q_i, K_i, V_i, followed by the row-parallel W_O shard, summed over
    shards, equals the unsharded attention block.  A head assigned to the wrong
    shard, a key head paired with the wrong query heads, or K and V swapped
    breaks the identity."""
    T, d = 6, 12
    rng = np.random.default_rng(Hq * 7 + Hkv * 3 + p)
    ncol = (Hq + 2 * Hkv) * dh
    X = rng.standard_normal((T, d))
    W = rng.standard_normal((d, ncol)) / math.sqrt(d)
    b = rng.standard_normal(ncol) * 0.1
    WO = rng.standard_normal((Hq * dh, d)) / math.sqrt(Hq * dh)
    full = X @ W + b
    Qf, Kf, Vf = full[:, :Hq * dh], full[:, Hq * dh:(Hq + Hkv) * dh], full[:, (Hq + Hkv) * dh:]
    ref = _heads_attention(Qf, Kf, Vf, Hq, Hkv, dh) @ WO
    qw, kw = Hq * dh // p, Hkv * dh // p
    parts = []
    for i in range(p):
        s = oracle.qkv_shard(X, W, Hq, Hkv, dh, i, p, bqkv=b)
        O = _heads_attention(s[:, :qw], s[:, qw:qw + kw], s[:, qw + kw:], Hq // p, Hkv // p, dh)
        parts.append(oracle.row_shard(O, WO, i, p))
    assert rel_fro(oracle.partial_sum(parts), ref) < 1e-12


def test_qkv_head_bookkeeping_one_hot(golden):
    """'What is Tensor Parallelism?', Llama 3.1 70B at TP = 8: each GPU gets 8
    query heads and 1 key/value head.  With X a one-hot row and weight column c
    holding the value c, the shard's output names the weight column behind each
    of its columns: the query columns must form whole heads, 8 of them, and the
    key and value columns one head each; over the 8 shards every head of every
    part appears exactly once, shard i's heads coming after shard i-1's."""
    g = golden("attention_head_split.txt")
    Hq, Hkv, p = int(g["llama_heads"]), int(g["llama_kv_heads"]), int(g["llama_tp"])
    dh = int(g["llama_hidden"]) // Hq
    ncol = (Hq + 2 * Hkv) * dh
    d = 3
    X = np.array([[0.0, 1.0, 0.0]])
    W = np.zeros((d, ncol))
    W[1, :] = np.arange(ncol, dtype=np.float64)
    seen = {"q": [], "k": [], "v": []}
    bounds = {"q": (0, Hq * dh), "k": (Hq * dh, (Hq + Hkv) * dh), "v": ((Hq + Hkv) * dh, ncol)}
    for i in range(p):
        cols = oracle.qkv_shard(X, W, Hq, Hkv, dh, i, p)[0].astype(np.int64)
        assert cols.shape == ((int(g["llama_q_heads_per_gpu"]) + 2 * int(g["llama_kv_heads_per_gpu"]))
                              * dh,)
        nq = int(g["llama_q_heads_per_gpu"]) * dh
        nk = int(g["llama_kv_heads_per_gpu"]) * dh
        for part, seg in (("q", cols[:nq]), ("k", cols[nq:nq + nk]), ("v", cols[nq + nk:])):
            lo, hi = bounds[part]
            assert ((seg >= lo) & (seg < hi)).all()
            rel = seg - lo
            heads = rel.reshape(-1, dh)
            # whole heads: each row of dh columns is one head's columns in order
            assert (heads == heads[:, :1] + np.arange(dh)).all() and (heads[:, 0] % dh == 0).all()
            seen[part].extend((heads[:, 0] // dh).tolist())
    for part, n in (("q", Hq), ("k", Hkv), ("v", Hkv)):
        assert seen[part] == list(range(n))


def test_attention_split_shapes(golden):
    """The shard shapes the pages print: Part 9's [4096, 3 x 1024] QKV shard and
    [1024, 4096] output-projection shard at 32 heads on 4 GPUs; initnode's 16
    heads per GPU at 64 heads and TP = 4."""
    g = golden("attention_head_split.txt")
    H, p, E = int(g["gpt_heads"]), int(g["gpt_tp"]), int(g["gpt_embed"])
    dh = E // H
    assert H // p == int(g["gpt_heads_per_gpu"])
    d = 8  # a narrow input; the shard width does not depend on it
    s = oracle.qkv_shard(np.ones((1, d)), np.zeros((d, 3 * E)), H, H, dh, p - 1, p)
    assert s.shape[1] == int(g["gpt_qkv_shard_cols"])
    # W_O is a row-parallel linear over the head columns: shard rows E / p
    Z = oracle.row_shard(np.ones((1, E // p)), np.zeros((E, E)), p - 1, p)
    assert (E // p, Z.shape[1]) == (int(g["gpt_out_shard_rows"]), int(g["gpt_out_shard_cols"]))
    H4, p4 = int(g["initnode_heads"]), int(g["initnode_tp"])
    s4 = oracle.qkv_shard(np.ones((1, d)), np.zeros((d, 3 * H4 * 2)), H4, H4, 2, 0, p4)
    assert s4.shape[1] == 3 * int(g["initnode_heads_per_gpu"]) * 2


def test_qkv_divisibility_errors():
    """Head counts must be divisible by the TP degree ('Tensor Parallelism
    Explained', section 4; Part 9's module asserts it)."""
    X = np.zeros((1, 4))
    with pytest.raises(ValueError):
        oracle.qkv_shard(X, np.zeros((4, 6 * 2)), 4, 1, 2, 0, 2)   # Hkv = 1 on 2 GPUs
    with pytest.raises(ValueError):
        oracle.qkv_shard(X, np.zeros((4, 9 * 2)), 3, 3, 2, 0, 2)   # Hq = 3 on 2 GPUs
    with pytest.raises(ValueError):
        oracle.qkv_shard(X, np.zeros((4, 12 * 2)), 4, 4, 2, 2, 2)  # i outside [0, p)


# ---------------------------------------------------------------- P-11 -------
# The backward pass of the shard: the column-parallel step's input gradient is
# a sum over the shards (what the all-reduce before the block adds up), the
# row-parallel step's is local ('Transformer math: tensor parallel', sections
# on the column- and row-parallel splits and the f and g operators).
def _bw_case(T, d, k, seed, gated, bias):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, d))
    W1 = rng.standard_normal((d, k)) / math.sqrt(d)
    Wu = rng.standard_normal((d, k)) / math.sqrt(d) if gated else None
    b1 = rng.standard_normal(k) * 0.5 if bias else None
    W2 = rng.standard_normal((k, d)) / math.sqrt(k)
    dZ = rng.standard_normal((T, d))
    return X, W1, Wu, b1, W2, dZ


def _assemble(X, W1, W2, dZ, p, act, b1=None, Wu=None):
    """Full-matrix gradients from the p shards: dX summed, weight blocks placed."""
    T, d = X.shape
    k = W1.shape[1]
    s = k // p
    g = {"dX": np.zeros((T, d)), "dW1": np.zeros((d, k)), "dW2": np.zeros((k, d))}
    if Wu is not None:
        g["dWu"] = np.zeros((d, k))
    if b1 is not None:
        g["db1"] = np.zeros(k)
    parts = []
    for i in range(p):
        o = oracle.mlp_shard_backward(X, W1, W2, dZ, i, p, act, b1=b1, Wu=Wu)
        parts.append(o["dXp"])
        g["dW1"][:, i * s:(i + 1) * s] = o["dW1"]
        g["dW2"][i * s:(i + 1) * s] = o["dW2"]
        if Wu is not None:
            g["dWu"][:, i * s:(i + 1) * s] = o["dWu"]
        if b1 is not None:
            g["db1"][i * s:(i + 1) * s] = o["db1"]
    g["dX"] = oracle.partial_sum(parts)
    return g


@pytest.mark.parametrize("act", ["gelu_tanh", "gelu_erf", "relu", "none", "swiglu"])
@pytest.mark.parametrize("p", [1, 2, 4])
def test_backward_finite_differences(act, p):
    """Central differences of L = sum(dZ * Z), Z from the forward oracle, against
    the assembled shard gradients for every input and weight entry."""
    gated = act == "swiglu"
    X, W1, Wu, b1, W2, dZ = _bw_case(3, 5, 8, 17 + p, gated, not gated)
    g = _assemble(X, W1, W2, dZ, p, act, b1=b1, Wu=Wu)

    def loss(X, W1, Wu, b1, W2):
        return float(np.sum(dZ * oracle.mlp_unsharded(X, W1, W2, act, b1=b1, Wu=Wu)))

    args = {"X": X, "W1": W1, "W2": W2}
    if gated:
        args["Wu"] = Wu
    else:
        args["b1"] = b1
    h = 1e-6
    for name, arr in args.items():
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            kw = {key: v.copy() for key, v in args.items()}
            kw[name][idx] += h
            up = loss(kw["X"], kw["W1"], kw.get("Wu"), kw.get("b1"), kw["W2"])
            kw[name][idx] -= 2 * h
            dn = loss(kw["X"], kw["W1"], kw.get("Wu"), kw.get("b1"), kw["W2"])
            num[idx] = (up - dn) / (2 * h)
        ana = g["d" + name]
        err = np.max(np.abs(num - ana)) / max(np.max(np.abs(ana)), 1e-300)
        assert err < 1e-6, (name, err)


@pytest.mark.parametrize("act", ["gelu_tanh", "gelu_erf", "relu", "swiglu"])
def test_backward_against_torch_autograd(act):
    """torch's fp64 CPU autograd (its own GeLU, SiLU and ReLU) on the unsharded
    block agrees with the assembled shard gradients."""
    gated = act == "swiglu"
    X, W1, Wu, b1, W2, dZ = _bw_case(6, 16, 32, 5, gated, not gated)
    g = _assemble(X, W1, W2, dZ, 4, act, b1=b1, Wu=Wu)
    t = {n: torch.tensor(v, dtype=torch.float64, requires_grad=True)
         for n, v in (("X", X), ("W1", W1), ("W2", W2), ("Wu", Wu), ("b1", b1)) if v is not None}
    F = torch.nn.functional
    if gated:
        Hh = F.silu(t["X"] @ t["W1"]) * (t["X"] @ t["Wu"])
    else:
        pre = t["X"] @ t["W1"] + t["b1"]
        Hh = {"gelu_tanh": lambda x: F.gelu(x, approximate="tanh"), "gelu_erf": F.gelu,
              "relu": F.relu}[act](pre)
    Z = Hh @ t["W2"]
    (Z * torch.tensor(dZ)).sum().backward()
    for n, v in t.items():
        assert rel_fro(g["d" + n], v.grad.numpy()) < 1e-12, n


def test_backward_linear_closed_form():
    """With no activation: dX = dZ (W1 W2)^T, dW1 = X^T dZ W2^T, dW2 = (X W1 + b1)^T dZ,
    db1 = column sums of dZ W2^T (numpy)."""
    X, W1, _, b1, W2, dZ = _bw_case(7, 12, 24, 9, False, True)
    g = _assemble(X, W1, W2, dZ, 3, "none", b1=b1)
    assert rel_fro(g["dX"], dZ @ (W1 @ W2).T) < 1e-12
    assert rel_fro(g["dW1"], X.T @ (dZ @ W2.T)) < 1e-12
    assert rel_fro(g["dW2"], (X @ W1 + b1).T @ dZ) < 1e-12
    assert rel_fro(g["db1"], (dZ @ W2.T).sum(axis=0)) < 1e-12


@pytest.mark.parametrize("T,d,k,p", [(1, 2, 2, 1), (2, 3, 4, 2), (3, 2, 6, 3)])
def test_backward_brute_force_exact_relu(T, d, k, p):
    """Exact rationals on small integers with ReLU (derivative 1 above 0, else 0):
    every gradient entry is an exact integer."""
    rng = np.random.default_rng(T * 10 + k)
    X = rng.integers(-3, 4, (T, d))
    W1 = rng.integers(-3, 4, (d, k))
    b1 = rng.integers(-2, 3, (k,))
    W2 = rng.integers(-3, 4, (k, d))
    dZ = rng.integers(-3, 4, (T, d))
    F = Fraction
    H = [[sum(F(int(X[t, c])) * int(W1[c, j]) for c in range(d)) + int(b1[j]) for j in range(k)]
         for t in range(T)]
    Y = [[max(h, F(0)) for h in row] for row in H]
    dY = [[sum(F(int(dZ[t, n])) * int(W2[j, n]) for n in range(d)) for j in range(k)]
          for t in range(T)]
    dH = [[dY[t][j] if H[t][j] > 0 else F(0) for j in range(k)] for t in range(T)]
    dX = [[sum(dH[t][j] * int(W1[c, j]) for j in range(k)) for c in range(d)] for t in range(T)]
    dW1 = [[sum(int(X[t, c]) * dH[t][j] for t in range(T)) for j in range(k)] for c in range(d)]
    dW2 = [[sum(Y[t][j] * int(dZ[t, n]) for t in range(T)) for n in range(d)] for j in range(k)]
    db1 = [sum(dH[t][j] for t in range(T)) for j in range(k)]
    g = _assemble(X.astype(float), W1.astype(float), W2.astype(float), dZ.astype(float), p,
                  "relu", b1=b1.astype(float))
    assert np.array_equal(g["dX"], np.array(dX, dtype=float))
    assert np.array_equal(g["dW1"], np.array(dW1, dtype=float))
    assert np.array_equal(g["dW2"], np.array(dW2, dtype=float))
    assert np.array_equal(g["db1"], np.array(db1, dtype=float))


@pytest.mark.parametrize("act", ["gelu_tanh", "swiglu"])
def test_backward_shard_blocks_equal_unsharded(act):
    """Each shard's weight-gradient block, and its columns of dH, are exactly the
    corresponding block of the p = 1 result (the same sums in the same order);
    the sum of the shards' dX terms equals the p = 1 dX up to reassociation."""
    gated = act == "swiglu"
    X, W1, Wu, b1, W2, dZ = _bw_case(5, 12, 32, 3, gated, not gated)
    full = oracle.mlp_shard_backward(X, W1, W2, dZ, 0, 1, act, b1=b1, Wu=Wu)
    p, s = 4, 8
    parts = []
    for i in range(p):
        o = oracle.mlp_shard_backward(X, W1, W2, dZ, i, p, act, b1=b1, Wu=Wu)
        cols = slice(i * s, (i + 1) * s)
        assert np.array_equal(o["dW1"], full["dW1"][:, cols])
        assert np.array_equal(o["dW2"], full["dW2"][cols])
        assert np.array_equal(o["dH"][:, :s], full["dH"][:, cols])
        if gated:
            assert np.array_equal(o["dWu"], full["dWu"][:, cols])
            assert np.array_equal(o["dH"][:, s:], full["dH"][:, 32 + i * s:32 + (i + 1) * s])
        else:
            assert np.array_equal(o["db1"], full["db1"][cols])
        parts.append(o["dXp"])
    assert rel_fro(oracle.partial_sum(parts), full["dXp"]) < 1e-12


@pytest.mark.parametrize("act", ["gelu_tanh", "gelu_erf", "swiglu", "relu", "none"])
def test_activation_derivatives(act):
    """act' against central differences of the forward activation, and against
    torch's fp64 autograd of its own GeLU / SiLU / ReLU."""
    x = np.concatenate([np.linspace(-10, 10, 401), [-1e-3, 1e-3, 0.5, -0.5]])
    if act == "relu":
        x = x[np.abs(x) > 1e-2]
    h = 1e-6
    num = (oracle.activation(act, x + h) - oracle.activation(act, x - h)) / (2 * h)
    ana = oracle.dactivation(act, x)
    assert np.max(np.abs(num - ana)) < 1e-8
    tx = torch.tensor(x, requires_grad=True)
    F = torch.nn.functional
    f = {"gelu_tanh": lambda v: F.gelu(v, approximate="tanh"), "gelu_erf": F.gelu,
         "swiglu": F.silu, "relu": F.relu, "none": lambda v: v * 1.0}[act]
    f(tx).sum().backward()
    assert np.max(np.abs(tx.grad.numpy() - ana)) < 1e-14
    if act == "relu":
        assert oracle.dactivation("relu", np.array([0.0]))[0] == 0.0


# ---------------------------------------------------------------- P-12 -------
# The attention core between the projections: per-head softmax(Q K^T / sqrt(dk)) V
# ('Transformer math: tensor parallel', section "Attention: parallel across heads"),
# causal in the GPT module of 'Building GPT from Scratch, Part 9'.
def _qkv(T, Hq, Hkv, dh, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, Hq * dh)) * scale, rng.standard_normal((T, Hkv * dh)) * scale,
            rng.standard_normal((T, Hkv * dh)))


@pytest.mark.parametrize("Hq,Hkv,causal,S", [(4, 4, True, 12), (8, 2, True, 6), (6, 3, False, 4),
                                             (4, 1, False, 12)])
def test_attention_against_torch_sdpa(Hq, Hkv, causal, S):
    """torch's fp64 scaled_dot_product_attention (key/value heads repeated for the
    grouped case), per sequence."""
    T, dh = 12, 8
    Q, K, V = _qkv(T, Hq, Hkv, dh, Hq * 10 + Hkv)
    O = oracle.attention(Q, K, V, Hq, Hkv, dh, causal=causal, S=S)
    g = Hq // Hkv
    for b in range(T // S):
        rows = slice(b * S, (b + 1) * S)
        q = torch.tensor(Q[rows]).reshape(S, Hq, dh).transpose(0, 1)
        k = torch.tensor(K[rows]).reshape(S, Hkv, dh).transpose(0, 1).repeat_interleave(g, dim=0)
        v = torch.tensor(V[rows]).reshape(S, Hkv, dh).transpose(0, 1).repeat_interleave(g, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal)
        ref = ref.transpose(0, 1).reshape(S, Hq * dh).numpy()
        assert rel_fro(O[rows], ref) < 1e-12


def test_attention_special_cases():
    """The first token of a causal sequence sees only itself (output = its value
    row); equal keys give the plain mean of the visible values; one key far above
    the others takes all the weight."""
    T, H, dh = 6, 2, 4
    Q, K, V = _qkv(T, H, H, dh, 3)
    O = oracle.attention(Q, K, V, H, H, dh, causal=True)
    assert np.array_equal(O[0], V[0])
    Ke = np.tile(K[:1], (T, 1))
    Oe = oracle.attention(Q, Ke, V, H, H, dh, causal=True)
    for t in range(T):
        assert np.allclose(Oe[t], V[:t + 1].mean(axis=0), rtol=0, atol=1e-12)
    Qs = np.ones((T, H * dh))
    Ks = np.zeros((T, H * dh))
    Ks[2] = 100.0
    Os = oracle.attention(Qs, Ks, V, H, H, dh, causal=False)
    assert np.allclose(Os, np.tile(V[2], (T, 1)), rtol=0, atol=1e-12)


def test_attention_scale_and_key_order():
    """Scores are scaled by 1/sqrt(dh) (doubling Q and K is the same as quartering
    the temperature); without the causal mask the order of the keys does not
    matter."""
    T, H, dh = 7, 3, 16
    Q, K, V = _qkv(T, H, H, dh, 11)
    O = oracle.attention(Q, K, V, H, H, dh, causal=False)
    perm = np.random.default_rng(1).permutation(T)
    assert rel_fro(oracle.attention(Q, K[perm], V[perm], H, H, dh, causal=False), O) < 1e-13
    # plain definition at dh = 16 for one row of one head (numpy), via the scale
    s = Q[3, :dh] @ K[:, :dh].T / 4.0
    w = np.exp(s - s.max())
    assert np.allclose(O[3, :dh], (w / w.sum()) @ V[:, :dh], rtol=0, atol=1e-13)


def test_attention_heads_split_across_shards():
    """Head shards: the attention of shard i's heads (its query and key/value
    column blocks) is exactly shard i's block of the unsharded attention."""
    T, Hq, Hkv, dh, p = 9, 8, 4, 4, 4
    Q, K, V = _qkv(T, Hq, Hkv, dh, 21)
    O = oracle.attention(Q, K, V, Hq, Hkv, dh)
    qw, kw = Hq * dh // p, Hkv * dh // p
    for i in range(p):
        Oi = oracle.attention(Q[:, i * qw:(i + 1) * qw], K[:, i * kw:(i + 1) * kw],
                              V[:, i * kw:(i + 1) * kw], Hq // p, Hkv // p, dh)
        assert np.array_equal(Oi, O[:, i * qw:(i + 1) * qw])


# ---------------------------------------------------------------- P-13 -------
# One pre-LayerNorm transformer block ('Building GPT from Scratch, Part 9',
# section "Communication Pattern per Transformer Block": LayerNorm, attention
# split by heads, residual, LayerNorm, FFN, residual; two reductions).
@pytest.mark.parametrize("T,d,eps", [(5, 16, 1e-5), (3, 7, 1e-3), (4, 64, 1e-6)])
def test_layernorm_against_torch(T, d, eps):
    """torch's fp64 layer_norm (biased variance, scale and shift)."""
    rng = np.random.default_rng(T * d)
    X = rng.standard_normal((T, d)) * 3 + 1
    g, b = rng.standard_normal(d), rng.standard_normal(d)
    ref = torch.nn.functional.layer_norm(torch.tensor(X), (d,), torch.tensor(g), torch.tensor(b),
                                         eps=eps).numpy()
    assert np.abs(oracle.layernorm(X, g, b, eps) - ref).max() < 1e-12


def test_layernorm_closed_forms():
    """A constant row maps to beta exactly; the row (a, -a) maps to
    +-a / sqrt(a^2 + eps) * gamma + beta."""
    g, b = np.array([2.0, -3.0]), np.array([0.5, 0.25])
    Y = oracle.layernorm(np.array([[7.0, 7.0], [1.5, -1.5]]), g, b, eps=0.25)
    assert np.array_equal(Y[0], b)
    r = 1.5 / math.sqrt(1.5 ** 2 + 0.25)
    assert np.allclose(Y[1], [r * 2.0 + 0.5, -r * -3.0 + 0.25], rtol=0, atol=1e-15)


def _block_params(d, Hq, Hkv, dh, k, act, seed, bias=True):
    rng = np.random.default_rng(seed)
    ncol = (Hq + 2 * Hkv) * dh
    P = dict(ln1=(rng.standard_normal(d), rng.standard_normal(d)),
             ln2=(rng.standard_normal(d), rng.standard_normal(d)),
             Wqkv=rng.standard_normal((d, ncol)) / math.sqrt(d),
             WO=rng.standard_normal((Hq * dh, d)) / math.sqrt(Hq * dh),
             W1=rng.standard_normal((d, k)) / math.sqrt(d),
             W2=rng.standard_normal((k, d)) / math.sqrt(k))
    if act == "swiglu":
        P["Wu"] = rng.standard_normal((d, k)) / math.sqrt(d)
    if bias:
        P.update(bqkv=rng.standard_normal(ncol), bO=rng.standard_normal(d), b2=rng.standard_normal(d))
        if act != "swiglu":
            P["b1"] = rng.standard_normal(k)
    return P


def _torch_block(X, Hq, Hkv, dh, act, S, causal, eps, P, mirror=False):
    """The same block from torch's fp64 library routines (layer_norm, matmul,
    scaled_dot_product_attention, gelu, silu, relu); with mirror, the stored
    activations go through torch's fp32 -> bf16 conversion."""
    t = lambda a: None if a is None else torch.tensor(a)  # noqa: E731
    q16 = (lambda a: a.float().bfloat16().double()) if mirror else (lambda a: a)  # noqa: E731
    X = t(X)
    T, d = X.shape
    g = Hq // Hkv
    ln = lambda x, gb: torch.nn.functional.layer_norm(x, (d,), t(gb[0]), t(gb[1]), eps=eps)  # noqa
    A = q16(ln(X, P["ln1"]))
    qkv = q16(A @ t(P["Wqkv"]) + (t(P["bqkv"]) if "bqkv" in P else 0))
    q, kk, v = qkv[:, :Hq * dh], qkv[:, Hq * dh:(Hq + Hkv) * dh], qkv[:, (Hq + Hkv) * dh:]
    O = torch.empty(T, Hq * dh, dtype=torch.float64)
    for b in range(T // S):
        r = slice(b * S, (b + 1) * S)
        qh = q[r].reshape(S, Hq, dh).transpose(0, 1)
        kh = kk[r].reshape(S, Hkv, dh).transpose(0, 1).repeat_interleave(g, dim=0)
        vh = v[r].reshape(S, Hkv, dh).transpose(0, 1).repeat_interleave(g, dim=0)
        o = torch.nn.functional.scaled_dot_product_attention(qh, kh, vh, is_causal=causal)
        O[r] = o.transpose(0, 1).reshape(S, Hq * dh)
    X1 = X + (q16(O) @ t(P["WO"]) + (t(P["bO"]) if "bO" in P else 0))
    B = q16(ln(X1, P["ln2"]))
    H = B @ t(P["W1"])
    if act == "swiglu":
        H = torch.nn.functional.silu(H) * (B @ t(P["Wu"]))
    else:
        H = H + (t(P["b1"]) if "b1" in P else 0)
        H = {"gelu_tanh": lambda x: torch.nn.functional.gelu(x, approximate="tanh"),
             "gelu_erf": torch.nn.functional.gelu, "relu": torch.relu,
             "none": lambda x: x}[act](H)
    return (X1 + (q16(H) @ t(P["W2"]) + (t(P["b2"]) if "b2" in P else 0))).numpy()


@pytest.mark.parametrize("T,S,Hq,Hkv,act,causal", [(12, 12, 4, 2, "gelu_tanh", True),
                                                   (10, 5, 2, 1, "swiglu", True),
                                                   (8, 4, 4, 4, "gelu_erf", False),
                                                   (6, 6, 2, 2, "relu", True)])
def test_block_against_torch(T, S, Hq, Hkv, act, causal):
    d, dh, k = 16, 4, 24
    P = _block_params(d, Hq, Hkv, dh, k, act, T * 7 + Hq)
    X = np.random.default_rng(T).standard_normal((T, d))
    out = oracle.block(X, Hq, Hkv, dh, act, S=S, causal=causal, eps=1e-5, **P)
    ref = _torch_block(X, Hq, Hkv, dh, act, S, causal, 1e-5, P)
    assert rel_fro(out, ref) < 1e-12


def test_block_residual_passthrough_and_rows():
    """With zero output projections and no biases after them the block returns its
    input exactly (both residual paths carry X through); the rows option gives
    exactly those rows of the full result."""
    d, Hq, Hkv, dh, k, T = 16, 4, 2, 4, 24, 9
    P = _block_params(d, Hq, Hkv, dh, k, "gelu_tanh", 3)
    X = np.random.default_rng(5).standard_normal((T, d))
    Z = dict(P, WO=np.zeros_like(P["WO"]), W2=np.zeros_like(P["W2"]), bO=np.zeros(d), b2=np.zeros(d))
    assert np.array_equal(oracle.block(X, Hq, Hkv, dh, "gelu_tanh", **Z), X)
    full = oracle.block(X, Hq, Hkv, dh, "gelu_tanh", **P)
    rows = [8, 0, 3]
    assert np.array_equal(oracle.block(X, Hq, Hkv, dh, "gelu_tanh", rows=rows, **P), full[rows])


@pytest.mark.parametrize("act,p", [("gelu_tanh", 2), ("swiglu", 4)])
def test_block_equals_its_tensor_parallel_split(act, p):
    """The block computed shard by shard — per shard its heads' QKV columns, the
    attention of those heads, the W_O row block, then the sum of the partials; the
    MLP shards likewise — equals the unsharded block (the two reductions of the
    page's communication pattern)."""
    d, Hq, Hkv, dh, k, T = 16, 8, 4, 4, 32, 7
    P = _block_params(d, Hq, Hkv, dh, k, act, 11)
    X = np.random.default_rng(13).standard_normal((T, d))
    A = oracle.layernorm(X, *P["ln1"])
    qw, kw = Hq * dh // p, Hkv * dh // p
    parts = []
    for i in range(p):
        qkv = oracle.qkv_shard(A, P["Wqkv"], Hq, Hkv, dh, i, p, bqkv=P["bqkv"])
        Oi = oracle.attention(qkv[:, :qw], qkv[:, qw:qw + kw], qkv[:, qw + kw:], Hq // p, Hkv // p, dh)
        parts.append(oracle.row_shard(Oi, P["WO"], i, p))
    X1 = X + oracle.partial_sum(parts, P["bO"])
    B = oracle.layernorm(X1, *P["ln2"])
    parts = [oracle.mlp_shard(B, P["W1"], P["W2"], i, p, act, b1=P.get("b1"), Wu=P.get("Wu"))[1]
             for i in range(p)]
    out = X1 + oracle.partial_sum(parts, P["b2"])
    assert rel_fro(out, oracle.block(X, Hq, Hkv, dh, act, **P)) < 1e-12


def test_round_bf16_against_torch():
    """The oracle's round-to-nearest-even bf16 (through fp32) equals torch's
    conversion, on random values over many binades, exact ties and specials."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal(20000) * np.exp2(rng.integers(-60, 60, 20000))
    ties = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 2.0 ** -130, 0.0,
                     -0.0, 3.3895313892515355e38, np.inf, -np.inf])
    x = np.concatenate([x, ties])
    ref = torch.tensor(x).float().bfloat16().double().numpy()
    got = oracle.round_bf16(x)
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))


@pytest.mark.parametrize("act", ["gelu_tanh", "swiglu"])
def test_block_mirror_mode_against_torch(act):
    """Mirror mode (a diagnostic) rounds exactly the stored activations: it equals
    the torch composition with torch's bf16 conversion at the same points, and it
    differs from the exact block."""
    T, S, Hq, Hkv, d, dh, k = 10, 5, 4, 2, 16, 4, 24
    P = _block_params(d, Hq, Hkv, dh, k, act, 77)
    X = np.random.default_rng(78).standard_normal((T, d))
    got = oracle.block(X, Hq, Hkv, dh, act, S=S, mirror=True, **P)
    ref = _torch_block(X, Hq, Hkv, dh, act, S, True, 1e-5, P, mirror=True)
    assert rel_fro(got, ref) < 1e-12
    assert rel_fro(got, oracle.block(X, Hq, Hkv, dh, act, S=S, **P)) > 1e-5


# ---------------------------------------------------------- block error model ----
@pytest.mark.parametrize("act,causal,S", [("gelu_tanh", True, 5), ("swiglu", False, 10)])
def test_block_storage_error_composition(act, causal, S):
    """The error model's unperturbed composition is the block itself (equal to the
    oracle block and to torch's fp64 composition), for all rows and a row subset;
    with rel = 0 it reports no error."""
    T, Hq, Hkv, d, dh, k = 10, 4, 2, 16, 4, 24
    P = _block_params(d, Hq, Hkv, dh, k, act, 91)
    X = np.random.default_rng(92).standard_normal((T, d))
    ref = oracle.block(X, Hq, Hkv, dh, act, S=S, causal=causal, **P) - X
    U, ef, em = oracle.block_storage_error(X, Hq, Hkv, dh, act, S=S, causal=causal, rel=0.0, **P)
    assert rel_fro(U, ref) < 1e-13 and ef == 0.0 and em == 0.0
    ref_t = _torch_block(X, Hq, Hkv, dh, act, S, causal, 1e-5, P) - X
    assert rel_fro(U, ref_t) < 1e-12
    rows = [9, 2, 4]
    Ur, _, _ = oracle.block_storage_error(X, Hq, Hkv, dh, act, S=S, causal=causal, rows=rows,
                                          rel=0.0, **P)
    assert rel_fro(Ur, ref[rows]) < 1e-13


def test_block_storage_error_linear_closed_form():
    """With W_O = 0 the attention half adds only b_O, and with no activation the FFN
    is linear: U = B W1 W2 + b_O + b2 with B = LayerNorm(X + b_O).  To first order the
    model's perturbations of B (by B * rel * xi1) and of the hidden activation
    Y = B W1 (by Y * rel * xi2) change U by (B xi1 rel) W1 W2 + (Y xi2 rel) W2, whose
    expected squared norm for independent xi uniform on [-1, 1] (variance 1/3) is
    rel^2 / 3 * (sum_tc B_tc^2 ||(W1 W2)_c||^2 + sum_tj Y_tj^2 ||(W2)_j||^2).  The
    model's Monte Carlo estimate matches this expectation."""
    T, Hq, Hkv, d, dh, k = 64, 2, 1, 32, 8, 48
    P = _block_params(d, Hq, Hkv, dh, k, "none", 93)
    P["WO"] = np.zeros_like(P["WO"])
    P.pop("b1", None)
    X = np.random.default_rng(94).standard_normal((T, d))
    rel = 2.0 ** -8
    U, ef, _ = oracle.block_storage_error(X, Hq, Hkv, dh, "none", rel=rel, draws=16, seed=3, **P)
    B = oracle.layernorm(X + P["bO"], *P["ln2"])
    Y = B @ P["W1"]
    M = P["W1"] @ P["W2"]
    expect = rel ** 2 / 3.0 * (np.sum(B ** 2 * np.sum(M ** 2, axis=1)[None, :])
                               + np.sum(Y ** 2 * np.sum(P["W2"] ** 2, axis=1)[None, :]))
    got = (ef * np.linalg.norm(U)) ** 2
    assert abs(got / expect - 1.0) < 0.1, (got, expect)
    np.testing.assert_allclose(U, B @ M + P["bO"] + P["b2"], rtol=1e-12, atol=1e-12)


def test_block_storage_error_is_first_order():
    """Halving the relative perturbation halves the modelled error (the model stays
    in the linear regime of the block), and a different draw gives nearly the same
    figure (the estimate averages over every element of the update)."""
    T, S, Hq, Hkv, d, dh, k = 24, 12, 4, 2, 32, 8, 48
    P = _block_params(d, Hq, Hkv, dh, k, "swiglu", 95)
    X = np.random.default_rng(96).standard_normal((T, d))
    _, e1, _ = oracle.block_storage_error(X, Hq, Hkv, dh, "swiglu", S=S, rel=2.0 ** -8, **P)
    _, e2, _ = oracle.block_storage_error(X, Hq, Hkv, dh, "swiglu", S=S, rel=2.0 ** -9, **P)
    _, e3, _ = oracle.block_storage_error(X, Hq, Hkv, dh, "swiglu", S=S, rel=2.0 ** -8, seed=7, **P)
    assert e1 > 0 and abs(e2 / e1 - 0.5) < 0.02
    assert abs(e3 / e1 - 1.0) < 0.2
