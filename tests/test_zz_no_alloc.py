"""tp_mlp_shard_noalloc: the MLP shard with the library's static scratch instead
of a caller's workspace (for callers that cannot allocate), through the C ABI,
against tp_mlp_shard on the same inputs: two calls in a row, the second with
fewer tokens (the scratch keeps the first call's content), on the few-token
path that uses the scratch and on the tiled path that needs none."""
import pytest
import torch

import megatron_tensor_mlp_amd as tp
import oracle
from megatron_tensor_mlp_amd import synth
from tests.helpers import assert_bf16_close, f64, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def dev(t):
    return None if t is None else t.to(DEV)


def both(X, W1, W2, i, p, act, Wu=None, b1=None):
    T, d = X.shape
    s = W1.shape[1] // p
    out = []
    for fn in (tp.tp_mlp_shard, tp.tp_mlp_shard_noalloc):
        Y = torch.full((T, s), float("nan"), dtype=torch.bfloat16, device=DEV)
        Z = torch.full((T, d), float("nan"), dtype=torch.float32, device=DEV)
        fn(dev(X), dev(W1), dev(W2), i, p, Y, Z, act=act, Wu=dev(Wu), b1=dev(b1))
        out.append((Y, Z))
    torch.cuda.synchronize()
    return out


# (T first, T second, d, k, p, act)
CASES = [
    (64, 9, 1032, 4096, 4, "swiglu"),
    (33, 1, 264, 1024, 2, "gelu_tanh"),
    (300, 17, 264, 1024, 4, "swiglu"),
]


@pytest.mark.parametrize("T1,T2,d,k,p,act", CASES)
def test_noalloc_matches_workspace_entry_point(T1, T2, d, k, p, act):
    sw = act == "swiglu"
    X, W1, Wu, b1, W2 = synth.small_case(T1, d, k, 800 + T1, sw, bias=not sw)
    for T in (T1, T2):
        i = p - 1 if T == T1 else 0
        say(f"noalloc case T={T} d={d} k={k} p={p} act={act} i={i}")
        Xt = X[:T].contiguous()
        (Yw, Zw), (Yn, Zn) = both(Xt, W1, W2, i, p, act, Wu=Wu, b1=b1)
        # the same kernels with the same split-K order: identical bits
        assert torch.equal(Yn, Yw) and torch.equal(Zn, Zw)
        Yr, Zr = oracle.mlp_shard(f64(Xt), f64(W1), f64(W2), i, p, act,
                                  b1=None if b1 is None else f64(b1),
                                  Wu=None if Wu is None else f64(Wu))
        assert_bf16_close(Yn, Yr, "Y")
        assert_bf16_close(Zn, Zr, "Z")


def test_noalloc_llama_decode_shard():
    """The Llama-70B TP=8 decode shard (T = 64, then T = 1) from the static scratch."""
    Wg, Wu, W2 = (dev(t) for t in synth.llama_shard_weights())
    X = synth.llama_tokens(64)
    for T in (64, 1):
        say(f"noalloc llama decode T={T}")
        (Yw, Zw), (Yn, Zn) = both(X[:T].contiguous(), Wg, W2, 0, 1, "swiglu", Wu=Wu)
        assert torch.equal(Yn, Yw) and torch.equal(Zn, Zw)


def test_noalloc_where_the_workspace_entry_point_splits_k():
    """A shape whose tiled GEMMs tp_mlp_shard splits K (2 x 28 and 2 x 32 tiles,
    K = 8192 and 3584): the no-alloc entry point runs them unsplit, so the two
    agree within the bf16 tolerance, and each matches the oracle (sampled rows)."""
    T, d, k = 300, 8192, 3584
    assert tp.tp_workspace_bytes(torch.bfloat16, "swiglu", T, d, k, 1) > 0
    X, W1, Wu, _, W2 = synth.small_case(T, d, k, 1900, True, False)
    say(f"noalloc split-K shape T={T} d={d} k={k}")
    (Yw, Zw), (Yn, Zn) = both(X, W1, W2, 0, 1, "swiglu", Wu=Wu)
    assert_bf16_close(Yn, Yw, "Y vs workspace entry point")
    assert_bf16_close(Zn, Zw, "Z vs workspace entry point")
    rows = [0, 1, 127, 128, 255, 256, 299]
    Yr, Zr = oracle.mlp_shard(f64(X[rows]), f64(W1), f64(W2), 0, 1, "swiglu", Wu=f64(Wu))
    for Y, Z in ((Yw, Zw), (Yn, Zn)):
        assert_bf16_close(Y[rows], Yr, "Y")
        assert_bf16_close(Z[rows], Zr, "Z")
