"""GPU parity: the HIP path (called through the C ABI) against the CPU oracle on
the same seeded inputs.  Small cases span several tiles with ragged tails;
full-size workloads are checked on sampled token rows (rows are independent, so
the oracle computes exactly those rows from their inputs)."""
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


def run_shard(X, W1, W2, i, p, act, Wu=None, b1=None, ldpad=0):
    """Run tp_mlp_shard on the GPU; optionally with padded leading dimensions."""
    T, d = X.shape
    k = W1.shape[1]
    s = k // p

    def padded(t, rows, cols, dtype):
        buf = torch.full((rows, cols + ldpad), float("nan"), dtype=dtype, device=DEV)
        return buf[:, :cols]

    def put(t):
        if t is None or t.dim() != 2 or ldpad == 0:
            return dev(t)
        v = padded(t, t.shape[0], t.shape[1], t.dtype)
        v.copy_(t)
        return v

    Y = padded(None, T, s, X.dtype)
    Z = padded(None, T, d, torch.float32)
    tp.tp_mlp_shard(put(X), put(W1), put(W2), i, p, Y, Z, act=act, Wu=put(Wu), b1=dev(b1))
    torch.cuda.synchronize()
    return Y, Z


# --------------------------------------------------------------------- bf16 small
CASES = [
    # (T, d, k, p, act)  -- T > 64 takes the tiled path, T <= 64 the few-token path
    (300, 264, 1024, 4, "swiglu"),
    (300, 264, 1024, 4, "gelu_tanh"),
    (257, 520, 768, 2, "gelu_erf"),
    (513, 136, 512, 1, "relu"),
    (65, 256, 2048, 8, "none"),
    (1, 264, 1024, 4, "swiglu"),
    (3, 264, 1024, 4, "gelu_tanh"),
    (8, 520, 768, 2, "swiglu"),
    (17, 1032, 1536, 4, "gelu_erf"),
    (63, 264, 1024, 4, "relu"),
    (64, 4104, 2048, 2, "swiglu"),
]


@pytest.mark.parametrize("T,d,k,p,act", CASES)
def test_shard_bf16_small(T, d, k, p, act):
    sw = act == "swiglu"
    X, W1, Wu, b1, W2 = synth.small_case(T, d, k, 100 + T, sw, bias=not sw)
    for i in sorted({0, p - 1}):
        say(f"case T={T} d={d} k={k} p={p} act={act} i={i}")
        Y, Z = run_shard(X, W1, W2, i, p, act, Wu=Wu, b1=b1)
        Yr, Zr = oracle.mlp_shard(f64(X), f64(W1), f64(W2), i, p, act, b1=f64(b1) if b1 is not None
                                  else None, Wu=f64(Wu) if Wu is not None else None)
        assert_bf16_close(Y, Yr, "Y")
        assert_bf16_close(Z, Zr, "Z")


# Few-token path: shapes chosen for the split-K plan's corners (k-ranges per
# column block S, the token-block size, the k tail of a stage).
DECODE_CASES = [
    # (T, d, k, p, act, what)
    (3, 264, 16384, 1, "swiglu", "column step: 256 workgroups, S = 1 (gate+up pair); row step S ~ 74"),
    (20, 136, 32768, 1, "gelu_tanh", "column step: S = 1, no partials; row step S = 128"),
    (40, 520, 1000, 1, "relu", "64-row stages with a k tail (520, 1000 not multiples of 64)"),
    (16, 264, 1024, 4, "swiglu", "16 tokens: the largest single token block"),
    (17, 264, 1024, 4, "gelu_erf", "17 tokens: two token blocks"),
    (32, 264, 1024, 4, "swiglu", "32 tokens"),
    (33, 264, 1024, 4, "none", "33 tokens: four token blocks"),
]


@pytest.mark.parametrize("T,d,k,p,act,what", DECODE_CASES)
def test_decode_plan_corners(T, d, k, p, act, what):
    sw = act == "swiglu"
    X, W1, Wu, b1, W2 = synth.small_case(T, d, k, 300 + T, sw, bias=not sw)
    for i in sorted({0, p - 1}):
        say(f"decode case T={T} d={d} k={k} p={p} act={act} i={i}: {what}")
        Y, Z = run_shard(X, W1, W2, i, p, act, Wu=Wu, b1=b1)
        Yr, Zr = oracle.mlp_shard(f64(X), f64(W1), f64(W2), i, p, act, b1=f64(b1) if b1 is not None
                                  else None, Wu=f64(Wu) if Wu is not None else None)
        assert_bf16_close(Y, Yr, "Y")
        assert_bf16_close(Z, Zr, "Z")


def test_decode_counters_left_zero():
    """The split-K arrival counters (the first bytes of the workspace) are zero
    again after every few-token call."""
    T, d, k = 8, 1032, 4096
    X, W1, Wu, _, W2 = synth.small_case(T, d, k, 9, True, False)
    need = tp.tp_workspace_bytes(torch.bfloat16, "swiglu", T, d, k, 1)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    Y = torch.empty(T, k, dtype=torch.bfloat16, device=DEV)
    Z = torch.empty(T, d, device=DEV)
    for _ in range(3):
        tp.tp_mlp_shard(dev(X), dev(W1), dev(W2), 0, 1, Y, Z, act="swiglu", Wu=dev(Wu), ws=ws)
    torch.cuda.synchronize()
    assert int(ws[:256].view(torch.int32).abs().sum()) == 0


@pytest.mark.parametrize("T", [5, 300])
def test_padded_leading_dimensions(T):
    """Views with leading dimensions above the row width (padding filled with NaN)."""
    X, W1, Wu, _, W2 = synth.small_case(T, 264, 1024, 7, True, False)
    Y, Z = run_shard(X, W1, W2, 3, 4, "swiglu", Wu=Wu, ldpad=24)
    Yr, Zr = oracle.mlp_shard(f64(X), f64(W1), f64(W2), 3, 4, "swiglu", Wu=f64(Wu))
    assert_bf16_close(Y, Yr, "Y")
    assert_bf16_close(Z, Zr, "Z")


def one_hot_bf16(T, d, k, seed):
    rng = np.random.default_rng(seed)
    X = rng.integers(-120, 121, (T, d)).astype(np.float32)
    W1 = np.zeros((d, k), np.float32)
    W2 = np.zeros((k, d), np.float32)
    sg1 = rng.choice([-1.0, 1.0], k)
    sg2 = rng.choice([-1.0, 1.0], k)
    for g in range(k):
        W1[(7 * g + 3) % d, g] = sg1[g]
        W2[g, (5 * g + 1) % d] = sg2[g]
    b1 = rng.integers(-8, 9, (k,)).astype(np.float32)
    bf = lambda a: torch.from_numpy(a).to(torch.bfloat16)  # noqa: E731
    return bf(X), bf(W1), bf(W2), bf(b1)


@pytest.mark.parametrize("T", [5, 64, 300])
@pytest.mark.parametrize("act", ["relu", "none"])
def test_bookkeeping_exact(T, act):
    """One-hot integer weights: every Y_i and Z_i entry is a small integer, so the
    shard's columns/rows must be exactly the right ones (bit-exact check)."""
    d, k, p = 264, 1024, 4
    X, W1, W2, b1 = one_hot_bf16(T, d, k, T)
    for i in range(p):
        Y, Z = run_shard(X, W1, W2, i, p, act, b1=b1)
        Yr, Zr = oracle.mlp_shard(f64(X), f64(W1), f64(W2), i, p, act, b1=f64(b1))
        assert np.array_equal(f64(Y), Yr), f"Y shard {i}"
        assert np.array_equal(f64(Z), Zr), f"Z shard {i}"


def test_bookkeeping_swiglu_gross():
    """SwiGLU with one-hot weights: off-by-shard mistakes give gross errors."""
    T, d, k, p = 70, 264, 1024, 4
    X, W1, W2, _ = one_hot_bf16(T, d, k, 3)
    X = (X / 64).to(torch.bfloat16)
    Xu, Wu, _, _ = one_hot_bf16(T, d, k, 4)
    for i in range(p):
        Y, Z = run_shard(X, W1, W2, i, p, "swiglu", Wu=Wu)
        Yr, Zr = oracle.mlp_shard(f64(X), f64(W1), f64(W2), i, p, "swiglu", Wu=f64(Wu))
        assert_bf16_close(Y, Yr, f"Y shard {i}")
        assert_bf16_close(Z, Zr, f"Z shard {i}")


# --------------------------------------------------------------------- fp32 (Day 41)
def test_tiny_f32_simulated_p4():
    """Day 41 shapes in fp32 (x [4,512], W1 [512,2048], b1, W2 [2048,512], p = 4,
    GeLU tanh): every Y_i, Z_i and the reduced Z match the oracle, the GPU column
    concat equals the GPU unsharded column step bit-for-bit, and the reduction
    equals the oracle's fp32 left-to-right sum of the GPU partials bit-for-bit."""
    X, W1, b1, W2 = synth.tiny_f32_inputs()
    T, d, k, p = 4, 512, 2048, 4
    s = k // p
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731
    Y = torch.empty(p, T, s, device=DEV)
    Zp = torch.empty(p, T, d, device=DEV)
    Z = torch.empty(T, d, device=DEV)
    tp.tp_mlp_simulated(t(X), t(W1), t(W2), p, Y, Zp, Z, act="gelu_tanh", b1=t(b1))
    torch.cuda.synchronize()
    for i in range(p):
        Yr, Zr = oracle.mlp_shard(X, W1, W2, i, p, "gelu_tanh", b1=b1)
        assert_f32_close(Y[i], Yr, f"Y{i}")
        assert_f32_close(Zp[i], Zr, f"Z{i}")
    assert_f32_close(Z, oracle.mlp_unsharded(X, W1, W2, "gelu_tanh", b1=b1), "Z")
    # concat of shards == unsharded (p = 1), bit-exact, as the Day 41 post prints
    Yfull = torch.empty(T, k, device=DEV)
    tp.tp_col_linear(t(X), t(W1), 0, 1, Yfull, act="gelu_tanh", b1=t(b1))
    torch.cuda.synchronize()
    cat = torch.cat([Y[i] for i in range(p)], dim=1)
    assert float((cat - Yfull).abs().max()) == 0.0
    ref = oracle.partial_sum_f32([Zp[i].cpu().numpy() for i in range(p)])
    assert np.array_equal(Z.cpu().numpy(), ref)


# --------------------------------------------------------------------- partial sum
@pytest.mark.parametrize("p", [1, 3, 8, 17, 64])
@pytest.mark.parametrize("bias", [False, True])
def test_partial_sum_bit_exact(p, bias):
    T, d = 37, 1032
    parts = [torch.from_numpy(synth.gaussian_f32((T, d), 500 + q)).to(DEV) for q in range(p)]
    b2 = torch.from_numpy(synth.gaussian_f32((d,), 9)).to(DEV) if bias else None
    Z = torch.empty(T, d, device=DEV)
    tp.tp_partial_sum(parts, Z, b2=b2)
    torch.cuda.synchronize()
    ref = oracle.partial_sum_f32([q.cpu().numpy() for q in parts],
                                 b2.cpu().numpy() if bias else None)
    assert np.array_equal(Z.cpu().numpy(), ref)


def test_partial_sum_in_place_and_strided():
    T, d, p = 33, 520, 5
    base = torch.from_numpy(synth.gaussian_f32((p, T, d + 8), 77)).to(DEV)
    parts = [base[q, :, :d] for q in range(p)]
    ref = oracle.partial_sum_f32([q.cpu().numpy() for q in parts])
    tp.tp_partial_sum(parts, parts[0])  # in place into partial 0
    torch.cuda.synchronize()
    assert np.array_equal(parts[0].cpu().numpy(), ref)


# --------------------------------------------------------------------- errors / ws
def test_bad_degree_leaves_output_untouched():
    """'Tensor Parallelism Explained', section 4: a degree that does not divide the
    sharded dimension is an error; nothing is launched."""
    X, W1, _, b1, W2 = synth.small_case(8, 64, 320, 1, False, True)
    Y = torch.full((8, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    Z = torch.full((8, 64), 7.0, device=DEV)
    with pytest.raises(tp.TpError) as e:
        tp.tp_mlp_shard(dev(X), dev(W1), dev(W2), 0, 3, Y, Z, act="gelu_tanh", b1=dev(b1))
    assert e.value.name == "TP_ERR_NOT_DIVISIBLE"
    torch.cuda.synchronize()
    assert bool((Y == 7.0).all()) and bool((Z == 7.0).all())


def test_workspace_reuse_and_determinism():
    """One zeroed workspace serves consecutive few-token calls of different shapes
    (the arrival counters are left zero), and the split-K reduction is
    deterministic."""
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=DEV)
    outs = []
    for T, d, k, p in ((8, 1032, 4096, 2), (64, 520, 2048, 4), (8, 1032, 4096, 2)):
        X, W1, Wu, _, W2 = synth.small_case(T, d, k, 5 * T + d, True, False)
        s = k // p
        Y = torch.empty(T, s, dtype=torch.bfloat16, device=DEV)
        Z = torch.empty(T, d, device=DEV)
        tp.tp_mlp_shard(dev(X), dev(W1), dev(W2), 1, p, Y, Z, act="swiglu", Wu=dev(Wu), ws=ws)
        torch.cuda.synchronize()
        Yr, Zr = oracle.mlp_shard(f64(X), f64(W1), f64(W2), 1, p, "swiglu", Wu=f64(Wu))
        assert_bf16_close(Y, Yr, "Y")
        assert_bf16_close(Z, Zr, "Z")
        outs.append(Z.cpu())
    assert torch.equal(outs[0], outs[2])


def test_zero_tokens():
    X = torch.empty(0, 64, dtype=torch.bfloat16, device=DEV)
    W1 = torch.zeros(64, 128, dtype=torch.bfloat16, device=DEV)
    W2 = torch.zeros(128, 64, dtype=torch.bfloat16, device=DEV)
    Y = torch.empty(0, 64, dtype=torch.bfloat16, device=DEV)
    Z = torch.empty(0, 64, device=DEV)
    tp.tp_mlp_shard(X, W1, W2, 1, 2, Y, Z, act="gelu_tanh")


# --------------------------------------------------------------------- full-size workloads
def sampled_rows(T, n):
    rows = {0, 1, T - 1, T // 2}
    for tile in (64, 128, 256):
        rows |= {min(T - 1, tile - 1), min(T - 1, tile)}
    rng = np.random.default_rng(T)
    rows |= set(rng.integers(0, T, max(0, n - len(rows))).tolist())
    return sorted(r for r in rows if 0 <= r < T)


# Tiled path, 256-row tiles: the small cases above have few tiles and take the
# 128-row configuration, so these shapes (more than 128 tiles of 256 rows, with
# ragged row and column tails) cover the 256-row kernels; rows are sampled.
TILE256_CASES = [
    # (T, d, k, act, what)
    (1000, 1032, 4296, "swiglu", "column step 4 x 34 tiles (ragged T and k)"),
    (1000, 520, 8504, "gelu_erf", "column step 4 x 34 tiles with bias"),
    (1000, 8456, 1024, "relu", "row step 4 x 34 tiles (ragged d)"),
]


@pytest.mark.parametrize("T,d,k,act,what", TILE256_CASES)
def test_tiled_256_rows_ragged(T, d, k, act, what):
    sw = act == "swiglu"
    X, W1, Wu, b1, W2 = synth.small_case(T, d, k, 500 + d, sw, bias=not sw)
    say(f"tiled-256 case T={T} d={d} k={k} act={act}: {what}")
    Y, Z = run_shard(X, W1, W2, 0, 1, act, Wu=Wu, b1=b1)
    rows = sampled_rows(T, 24)
    Yr, Zr = oracle.mlp_shard(f64(X[rows]), f64(W1), f64(W2), 0, 1, act,
                              b1=f64(b1) if b1 is not None else None,
                              Wu=f64(Wu) if Wu is not None else None)
    assert_bf16_close(Y[rows], Yr, "Y")
    assert_bf16_close(Z[rows], Zr, "Z")


# Tiled path with split K (few output tiles, long K): S k-ranges per tile meet
# in the workspace, where the last arriving workgroup sums them in order.
SPLIT_CASES = [
    # (T, d, k, p, act, what)
    (300, 8192, 3584, 1, "swiglu", "column 2 x 28 tiles, 4 k-ranges; row 2 x 32 tiles, 3 k-ranges"),
    (257, 4104, 2048, 1, "gelu_tanh",
     "column 2 x 8 tiles, 5 k-ranges (last 776 of 832); row 2 x 17 tiles, 2 k-ranges; bias"),
    (100, 3080, 512, 1, "relu", "column 1 x 2 tiles, 4 k-ranges (last 680 of 800), bias"),
    (65, 12296, 1024, 4, "none", "column one tile, 8 k-ranges (last 1320), bias"),
]


@pytest.mark.parametrize("T,d,k,p,act,what", SPLIT_CASES)
def test_tiled_split_k(T, d, k, p, act, what):
    sw = act == "swiglu"
    X, W1, Wu, b1, W2 = synth.small_case(T, d, k, 700 + T, sw, bias=not sw)
    i = p - 1
    say(f"split-K case T={T} d={d} k={k} p={p} act={act} i={i}: {what}")
    Y, Z = run_shard(X, W1, W2, i, p, act, Wu=Wu, b1=b1)
    rows = sampled_rows(T, 24)
    Yr, Zr = oracle.mlp_shard(f64(X[rows]), f64(W1), f64(W2), i, p, act,
                              b1=f64(b1) if b1 is not None else None,
                              Wu=f64(Wu) if Wu is not None else None)
    assert_bf16_close(Y[rows], Yr, "Y")
    assert_bf16_close(Z[rows], Zr, "Z")
    assert bool(torch.isfinite(Y).all()) and bool(torch.isfinite(Z).all())


def test_tiled_without_workspace_runs_unsplit():
    """With more than 64 tokens the split-K workspace is optional: given too
    little, the tiled GEMMs run unsplit and still match the oracle (and the
    split result within the bf16 tolerance); with 64 or fewer tokens a missing
    workspace is an error and nothing is written."""
    T, d, k = 300, 8192, 3584
    X, W1, Wu, _, W2 = synth.small_case(T, d, k, 1700, True, False)
    tiny = torch.zeros(16, dtype=torch.uint8, device=DEV)
    outs = []
    for ws in (tiny, None):  # unsplit, then split (the binding sizes the workspace)
        say(f"tiled T={T} d={d} k={k} with {'a 16-byte' if ws is not None else 'a full'} workspace")
        Y = torch.full((T, k), float("nan"), dtype=torch.bfloat16, device=DEV)
        Z = torch.full((T, d), float("nan"), device=DEV)
        tp.tp_mlp_shard(dev(X), dev(W1), dev(W2), 0, 1, Y, Z, act="swiglu", Wu=dev(Wu), ws=ws)
        torch.cuda.synchronize()
        outs.append((Y, Z))
    rows = sampled_rows(T, 16)
    Yr, Zr = oracle.mlp_shard(f64(X[rows]), f64(W1), f64(W2), 0, 1, "swiglu", Wu=f64(Wu))
    for Y, Z in outs:
        assert_bf16_close(Y[rows], Yr, "Y")
        assert_bf16_close(Z[rows], Zr, "Z")
    assert_bf16_close(outs[0][0], outs[1][0], "Y unsplit vs split")
    assert_bf16_close(outs[0][1], outs[1][1], "Z unsplit vs split")

    Xs, W1s, Wus, _, W2s = synth.small_case(8, 1032, 4096, 1701, True, False)
    Y = torch.full((8, 2048), 7.0, dtype=torch.bfloat16, device=DEV)
    Z = torch.full((8, 1032), 7.0, device=DEV)
    with pytest.raises(tp.TpError) as e:
        tp.tp_mlp_shard(dev(Xs), dev(W1s), dev(W2s), 1, 2, Y, Z, act="swiglu", Wu=dev(Wus), ws=tiny)
    assert e.value.name == "TP_ERR_WORKSPACE"
    torch.cuda.synchronize()
    assert bool((Y == 7.0).all()) and bool((Z == 7.0).all())


def test_split_k_workspace_reuse_and_determinism():
    """One zeroed workspace serves split-K tiled calls of two shapes and a
    few-token call in between; every call leaves the arrival counters zero, and
    the same call gives the same bits again."""
    ws = torch.zeros(96 << 20, dtype=torch.uint8, device=DEV)
    seq = [(300, 8192, 3584, 1, "swiglu"), (65, 12296, 1024, 4, "none"),
           (8, 1032, 4096, 2, "swiglu"), (300, 8192, 3584, 1, "swiglu")]
    data = {}
    outs = []
    for T, d, k, p, act in seq:
        sw = act == "swiglu"
        if (T, d, k) not in data:
            data[(T, d, k)] = synth.small_case(T, d, k, 900 + T, sw, bias=not sw)
        X, W1, Wu, b1, W2 = data[(T, d, k)]
        need = tp.tp_workspace_bytes(torch.bfloat16, act, T, d, k, p)
        assert 0 < need <= ws.numel()
        say(f"split-K reuse T={T} d={d} k={k} p={p} act={act}")
        Y = torch.empty(T, k // p, dtype=torch.bfloat16, device=DEV)
        Z = torch.empty(T, d, device=DEV)
        tp.tp_mlp_shard(dev(X), dev(W1), dev(W2), p - 1, p, Y, Z, act=act, Wu=dev(Wu),
                        b1=dev(b1), ws=ws)
        torch.cuda.synchronize()
        assert int(ws[:256 << 10].count_nonzero()) == 0
        outs.append((Y.cpu(), Z.cpu()))
    assert torch.equal(outs[0][0], outs[3][0]) and torch.equal(outs[0][1], outs[3][1])


def test_gpt_gelu_shard_full_size():
    """GPT-style GeLU shard at d = 4096, k/p = 4096 (compact shard), T = 2048."""
    W = synth.WORKLOADS["gpt_gelu_p4"]
    X, W1, b1, W2 = synth.gpt_gelu_shard_inputs(W.T, W.d, W.s)
    say(f"workload {W.name}: T={W.T} d={W.d} s={W.s}")
    Y, Z = run_shard(X, W1, W2, 0, 1, "gelu_tanh", b1=b1)
    rows = sampled_rows(W.T, 12)
    Yr, Zr = oracle.mlp_shard(f64(X[rows]), f64(W1), f64(W2), 0, 1, "gelu_tanh", b1=f64(b1))
    assert_bf16_close(Y[rows], Yr, "Y")
    assert_bf16_close(Z[rows], Zr, "Z")
    assert bool(torch.isfinite(Z).all())


def test_llama_prefill_shard_full_size():
    """Llama-70B SwiGLU shard at TP = 8 (d = 8192, k/p = 3584), T = 4096."""
    W = synth.WORKLOADS["llama70b_prefill_tp8"]
    Wg, Wu, W2 = synth.llama_shard_weights(W.d, W.s)
    X = synth.llama_tokens(W.T, W.d)
    say(f"workload {W.name}: T={W.T} d={W.d} s={W.s}")
    Y, Z = run_shard(X, Wg, W2, 0, 1, "swiglu", Wu=Wu)
    rows = sampled_rows(W.T, 10)
    Yr, Zr = oracle.mlp_shard(f64(X[rows]), f64(Wg), f64(W2), 0, 1, "swiglu", Wu=f64(Wu))
    assert_bf16_close(Y[rows], Yr, "Y")
    assert_bf16_close(Z[rows], Zr, "Z")
    assert bool(torch.isfinite(Z).all())


@pytest.mark.parametrize("T", [1, 8, 64])
def test_llama_decode_shard_full_size(T):
    """Llama-70B SwiGLU shard at TP = 8, few-token decode (all rows checked)."""
    W = synth.WORKLOADS["llama70b_decode_tp8"]
    Wg, Wu, W2 = synth.llama_shard_weights(W.d, W.s)
    X = synth.llama_tokens(T, W.d)
    say(f"workload {W.name}: T={T}")
    Y, Z = run_shard(X, Wg, W2, 0, 1, "swiglu", Wu=Wu)
    Yr, Zr = oracle.mlp_shard(f64(X), f64(Wg), f64(W2), 0, 1, "swiglu", Wu=f64(Wu))
    assert_bf16_close(Y, Yr, "Y")
    assert_bf16_close(Z, Zr, "Z")


def test_llama_block_simulated_tp8():
    """All 8 shards of a Llama-70B MLP (full [8192, 28672] weights, shards as views)
    on one GPU, then the on-device reduction, against the unsharded oracle."""
    W = synth.WORKLOADS["llama70b_block_sim_tp8"]
    Wg, Wu, W2 = synth.llama_full_weights(W.d, W.k)
    X = synth.llama_tokens(W.T, W.d)
    say(f"workload {W.name}: T={W.T} d={W.d} k={W.k} p={W.p}")
    Y = torch.empty(W.p, W.T, W.s, dtype=torch.bfloat16, device=DEV)
    Zp = torch.empty(W.p, W.T, W.d, device=DEV)
    Z = torch.empty(W.T, W.d, device=DEV)
    tp.tp_mlp_simulated(dev(X), dev(Wg), dev(W2), W.p, Y, Zp, Z, act="swiglu", Wu=dev(Wu))
    torch.cuda.synchronize()
    rows = [0, 255, 256, 511]
    Zr = oracle.mlp_unsharded(f64(X[rows]), f64(Wg), f64(W2), "swiglu", Wu=f64(Wu))
    assert_bf16_close(Z[rows], Zr, "Z")
    ref = oracle.partial_sum_f32([Zp[i].cpu().numpy() for i in range(W.p)])
    assert np.array_equal(Z.cpu().numpy(), ref)


# Simulated mode whose grouped column launch splits K: (T, d, k, p, act, what)
SIM_SPLIT_CASES = [
    (300, 8192, 1024, 4, "gelu_tanh", "4 groups x 2 tiles, 8 k-ranges, bias"),
    (300, 8192, 2048, 4, "swiglu", "4 groups x 2 x 4 tiles, 4 k-ranges"),
]


@pytest.mark.parametrize("T,d,k,p,act,what", SIM_SPLIT_CASES)
def test_simulated_split_k(T, d, k, p, act, what):
    """All p shards as grouped launches whose column step splits K, then the
    reduction: each shard's Y and the summed Z against the oracle on sampled
    rows, and Z bit for bit against the left-to-right sum of the partials."""
    sw = act == "swiglu"
    X, W1, Wu, b1, W2 = synth.small_case(T, d, k, 1100 + k, sw, bias=not sw)
    s = k // p
    say(f"simulated split-K case T={T} d={d} k={k} p={p} act={act}: {what}")
    Y = torch.empty(p, T, s, dtype=torch.bfloat16, device=DEV)
    Zp = torch.empty(p, T, d, device=DEV)
    Z = torch.empty(T, d, device=DEV)
    tp.tp_mlp_simulated(dev(X), dev(W1), dev(W2), p, Y, Zp, Z, act=act, Wu=dev(Wu), b1=dev(b1))
    torch.cuda.synchronize()
    rows = sampled_rows(T, 12)
    for i in range(p):
        Yr, Zr = oracle.mlp_shard(f64(X[rows]), f64(W1), f64(W2), i, p, act,
                                  b1=f64(b1) if b1 is not None else None,
                                  Wu=f64(Wu) if Wu is not None else None)
        assert_bf16_close(Y[i][rows], Yr, f"Y_{i}")
        assert_bf16_close(Zp[i][rows], Zr, f"Z_{i}")
    ref = oracle.partial_sum_f32([Zp[i].cpu().numpy() for i in range(p)])
    assert np.array_equal(Z.cpu().numpy(), ref)


@pytest.mark.parametrize("T,ldx", [(300, (1 << 21) - 8), (17, (1 << 23) - 8)])
def test_largest_supported_leading_dimension(T, ldx):
    """X as a view of a buffer with the largest leading dimension each path
    accepts (below 2^21 elements with more than 64 tokens, below 2^23 with 64 or
    fewer): the per-lane 32-bit offsets stay in range (NaN fills the rest)."""
    X, W1, Wu, _, W2 = synth.small_case(T, 264, 1024, 19, True, False)
    buf = torch.full((T, ldx), float("nan"), dtype=torch.bfloat16, device=DEV)
    buf[:, :264] = dev(X)
    Xv = buf[:, :264]
    s = 1024 // 4
    Y = torch.empty(T, s, dtype=torch.bfloat16, device=DEV)
    Z = torch.empty(T, 264, device=DEV)
    say(f"largest leading dimension: T={T} ldx={ldx}")
    tp.tp_mlp_shard(Xv, dev(W1), dev(W2), 2, 4, Y, Z, act="swiglu", Wu=dev(Wu))
    torch.cuda.synchronize()
    Yr, Zr = oracle.mlp_shard(f64(X), f64(W1), f64(W2), 2, 4, "swiglu", Wu=f64(Wu))
    assert_bf16_close(Y, Yr, "Y")
    assert_bf16_close(Z, Zr, "Z")
