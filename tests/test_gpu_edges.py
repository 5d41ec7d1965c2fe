"""GPU parity at the numeric edges of the method, through the C ABI, against the
CPU oracle on the same seeded inputs.

Attention ('Transformer math: tensor parallel', section 'Attention: parallel
across heads': each head computes softmax(Q K^T / sqrt(d_k)) V on its own):
scores with a standard deviation of 10 and 30, a score ramp that rises (or
falls) steadily along the sequence so that the running maximum moves in most
key tiles, and one dominant key per query.  These reach the core's rescaling
of the running sum and output (the reference maximum moves only when a tile
beats it by more than 2^8), its merge of two partial softmax states, and
weights that underflow to zero.

MLP ('Transformer math: tensor parallel', section 'The MLP block: column then
row'): pre-activations spanning about +-40 for every activation on both GEMM
paths, reaching GeLU's saturation and SiLU's exp overflow for large negative
inputs."""
import math

import numpy as np
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


def run_core(Q, K, V, Hq, Hkv, dh, S, causal):
    T = Q.shape[0]
    O = torch.full((T, Hq * dh + 8), float("nan"), dtype=torch.bfloat16, device=DEV)
    tp.tp_attention(dev(Q), dev(K), dev(V), O[:, :Hq * dh], Hq, Hkv, dh, S=S, causal=causal)
    torch.cuda.synchronize()
    assert bool(torch.isnan(O[:, Hq * dh:]).all())
    return O[:, :Hq * dh]


def score_spread(Q, K, Hq, Hkv, dh, S):
    """Standard deviation of q.k / sqrt(dh) over the first sequence (test-side
    statistics of the inputs, for the case description)."""
    q, k = f64(Q[:S]), f64(K[:S])
    grp = Hq // Hkv
    s = [q[:, h * dh:(h + 1) * dh] @ k[:, (h // grp) * dh:(h // grp + 1) * dh].T
         for h in range(Hq)]
    return float(np.std(np.stack(s)) / math.sqrt(dh))


# (nseq, S, Hq, Hkv, dh, causal, score_std)
SCALED = [
    (1, 300, 4, 2, 128, True, 10.0),
    (1, 300, 4, 2, 128, True, 30.0),
    (2, 200, 2, 2, 64, False, 10.0),
    (2, 200, 2, 2, 64, False, 30.0),
    (1, 576, 8, 1, 128, True, 30.0),
    (2, 129, 4, 1, 64, True, 20.0),
    (1, 333, 8, 4, 128, False, 30.0),
]


@pytest.mark.parametrize("nseq,S,Hq,Hkv,dh,causal,score_std", SCALED)
def test_attention_large_scores(nseq, S, Hq, Hkv, dh, causal, score_std):
    Q, K, V = synth.attn_scaled(nseq * S, Hq, Hkv, dh, 400 + S, score_std)
    sd = score_spread(Q, K, Hq, Hkv, dh, S)
    say(f"attention large scores nseq={nseq} S={S} Hq={Hq} Hkv={Hkv} dh={dh} causal={causal} "
        f"score std {sd:.1f}")
    assert 0.8 * score_std < sd < 1.2 * score_std
    O = run_core(Q, K, V, Hq, Hkv, dh, S, causal)
    ref = oracle.attention(f64(Q), f64(K), f64(V), Hq, Hkv, dh, causal=causal, S=S)
    assert_bf16_close(O, ref, "O")


# (nseq, S, Hq, Hkv, dh, causal, slope)
RAMPS = [
    (1, 576, 2, 1, 128, True, 0.02),
    (1, 576, 2, 1, 128, True, -0.02),
    (1, 576, 4, 2, 64, False, 0.03),
    (2, 333, 4, 4, 64, True, 0.03),
    (1, 1000, 8, 1, 128, True, 0.01),
    (2, 300, 2, 2, 128, False, -0.02),
]


@pytest.mark.parametrize("nseq,S,Hq,Hkv,dh,causal,slope", RAMPS)
def test_attention_score_ramp(nseq, S, Hq, Hkv, dh, causal, slope):
    """Key j's score moves by about sqrt(dh) * slope per key: more than 8 in
    base 2 per 64-key tile, so the reference maximum moves in most tiles a
    workgroup walks in ascending key order (rising ramp) or descending order
    (falling ramp, the second half of a block pair's tile list)."""
    Q, K, V = synth.attn_ramp(nseq, S, Hq, Hkv, dh, 500 + S, slope)
    per_tile = abs(math.sqrt(dh) * slope * 64) * math.log2(math.e)
    say(f"attention ramp nseq={nseq} S={S} Hq={Hq} Hkv={Hkv} dh={dh} causal={causal} "
        f"slope={slope}: ~{per_tile:.0f} (base 2) per key tile")
    assert per_tile > 8.0
    O = run_core(Q, K, V, Hq, Hkv, dh, S, causal)
    ref = oracle.attention(f64(Q), f64(K), f64(V), Hq, Hkv, dh, causal=causal, S=S)
    assert_bf16_close(O, ref, "O")


# (nseq, S, Hq, Hkv, dh, causal)
DOMINANT = [
    (1, 300, 4, 2, 128, True),
    (2, 257, 2, 1, 64, True),
    (1, 576, 8, 1, 128, True),
    (2, 200, 4, 4, 64, False),
    (1, 333, 8, 2, 128, False),
]


@pytest.mark.parametrize("nseq,S,Hq,Hkv,dh,causal", DOMINANT)
def test_attention_dominant_key(nseq, S, Hq, Hkv, dh, causal):
    """Every query has one key whose score is about 3 sqrt(dh) against N(0, 9)
    for the rest: the softmax puts practically all its weight there, so the
    output row is that key's value row (a closed form checked next to the
    oracle)."""
    Q, K, V, jstar = synth.attn_dominant(nseq, S, Hq, Hkv, dh, 600 + S, causal)
    say(f"attention dominant key nseq={nseq} S={S} Hq={Hq} Hkv={Hkv} dh={dh} causal={causal}")
    O = run_core(Q, K, V, Hq, Hkv, dh, S, causal)
    ref = oracle.attention(f64(Q), f64(K), f64(V), Hq, Hkv, dh, causal=causal, S=S)
    assert_bf16_close(O, ref, "O")
    T = nseq * S
    grp = Hq // Hkv
    rows = (np.arange(T) // S) * S
    v = f64(V)
    pick = np.concatenate([v[rows + jstar[:, h], (h // grp) * dh:(h // grp + 1) * dh]
                           for h in range(Hq)], axis=1)
    assert_bf16_close(O, pick, "O vs the dominant key's value row")


# ------------------------------------------------------------------------ MLP
# (T, d, k, p, act): T > 64 takes the tiled path, T <= 64 the few-token path.
WIDE = [(T, 264, 1024, 4, act) for T in (300, 17, 1)
        for act in ("gelu_tanh", "gelu_erf", "swiglu", "relu")]


@pytest.mark.parametrize("T,d,k,p,act", WIDE)
def test_mlp_preactivations_span_40(T, d, k, p, act):
    """Weights N(0, 1) instead of N(0, 0.02^2): the pre-activations have a
    standard deviation of about 16 and reach past +-40 in every case."""
    sw = act == "swiglu"
    X, W1, Wu, b1, W2 = synth.small_case(T, d, k, 700 + T, sw, bias=not sw, w_std=1.0)
    s = k // p
    for i in sorted({0, p - 1}):
        h = f64(X) @ f64(W1)[:, i * s:(i + 1) * s]
        say(f"wide pre-activation case T={T} act={act} i={i}: range [{h.min():.0f}, {h.max():.0f}]")
        if T > 1:
            assert h.min() < -40 and h.max() > 40
        Y = torch.empty(T, s, dtype=torch.bfloat16, device=DEV)
        Z = torch.empty(T, d, dtype=torch.float32, device=DEV)
        tp.tp_mlp_shard(dev(X), dev(W1), dev(W2), i, p, Y, Z, act=act, Wu=dev(Wu), b1=dev(b1))
        torch.cuda.synchronize()
        Yr, Zr = oracle.mlp_shard(f64(X), f64(W1), f64(W2), i, p, act,
                                  b1=None if b1 is None else f64(b1),
                                  Wu=None if Wu is None else f64(Wu))
        assert_bf16_close(Y, Yr, "Y")
        assert_bf16_close(Z, Zr, "Z")
