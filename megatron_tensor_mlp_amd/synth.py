"""Seeded synthetic inputs for the tensor-parallel MLP shard.

This module only draws numbers: shapes, seeds and value distributions of the
workloads.  It holds none of the method's arithmetic, so both the GPU path and
the CPU oracle can be fed from it without sharing any computation.

bf16 inputs are drawn in fp32 and rounded to bf16 (round to nearest even) by
torch; the GPU receives those bf16 values and the oracle receives the very same
values widened exactly to fp64.

Workload shapes come from the pages' worked examples:
  * the Day 41 post's fp32 check (x [4,512], W [512,2048], p = 4, seed 42);
  * a GPT-style d = 4096, d_ff = 16384 MLP split four ways ("Transformer math:
    tensor parallel", section "A worked example"; "Building GPT from Scratch,
    Part 9", section "Splitting the FFN Layer");
  * Llama 3.1 70B at TP = 8: hidden 8192, feed-forward 28672, 3584 feed-forward
    columns per GPU ("What is Tensor Parallelism?", section "Worked example:
    Llama 3.1 70B on 8 GPUs"), with the gated SwiGLU feed-forward ("Tensor
    Parallelism Explained", section 2.B);
  * attention split by heads: Llama 3.1 70B's 64 query and 8 key/value heads
    at TP = 8 (same page and section; head width 8192 / 64 = 128), and the
    GPT-style 32 heads of width 128 over 4 GPUs ("Building GPT from Scratch,
    Part 9", section "Splitting the Attention Layer").
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

WEIGHT_STD = 0.02


@dataclass(frozen=True)
class Workload:
    name: str
    T: int          # tokens
    d: int          # model width
    k: int          # full hidden width (d_ff)
    p: int          # tensor-parallel degree
    act: str        # "gelu_tanh" or "swiglu"
    dtype: str      # "f32" or "bf16"
    bias: bool      # column bias b1 present
    note: str = ""
    Ts: tuple = field(default_factory=tuple)  # decode: several token counts

    @property
    def s(self) -> int:
        return self.k // self.p

    @property
    def n_gemm(self) -> int:
        return 3 if self.act == "swiglu" else 2

    def shard_flops(self, T: int | None = None) -> float:
        """Algorithmic flops of one shard forward: 2*T*d*(k/p) per GEMM."""
        T = self.T if T is None else T
        return 2.0 * T * self.d * self.s * self.n_gemm


WORKLOADS = {
    "tiny_f32_p4": Workload("tiny_f32_p4", 4, 512, 2048, 4, "gelu_tanh", "f32", True,
                            "Day 41 post fp32 check shape, GeLU(tanh), p=4 simulated"),
    "gpt_gelu_p4": Workload("gpt_gelu_p4", 2048, 4096, 16384, 4, "gelu_tanh", "bf16", True,
                            "GPT-style GeLU MLP shard, p=4, zero bias"),
    "llama70b_prefill_tp8": Workload("llama70b_prefill_tp8", 4096, 8192, 28672, 8, "swiglu",
                                     "bf16", False, "Llama-70B SwiGLU shard, TP=8, prefill"),
    "llama70b_decode_tp8": Workload("llama70b_decode_tp8", 64, 8192, 28672, 8, "swiglu", "bf16",
                                    False, "Llama-70B SwiGLU shard, TP=8, decode",
                                    Ts=(1, 8, 64)),
    "llama70b_block_sim_tp8": Workload("llama70b_block_sim_tp8", 512, 8192, 28672, 8, "swiglu",
                                       "bf16", False,
                                       "all 8 shards of a TP=8 Llama-70B MLP on one GPU"),
}


@dataclass(frozen=True)
class AttnWorkload:
    """Attention projections of one head shard: QKV [d, (Hq + 2 Hkv) dh / p] and
    the output projection's row block [Hq dh / p, d]."""
    name: str
    T: int          # tokens
    d: int          # model width
    Hq: int         # query heads
    Hkv: int        # key/value heads
    dh: int         # head width
    p: int          # tensor-parallel degree
    note: str = ""
    Ts: tuple = field(default_factory=tuple)  # decode: several token counts

    @property
    def qkv_cols(self) -> int:
        return (self.Hq + 2 * self.Hkv) * self.dh // self.p

    @property
    def o_rows(self) -> int:
        return self.Hq * self.dh // self.p

    def shard_flops(self, T: int | None = None) -> float:
        """Algorithmic flops of the shard's two projections: 2 T d (qkv_cols + o_rows)."""
        T = self.T if T is None else T
        return 2.0 * T * self.d * (self.qkv_cols + self.o_rows)

    def weight_bytes(self) -> int:
        """bf16 bytes of the shard's two weight blocks."""
        return 2 * self.d * (self.qkv_cols + self.o_rows)


ATTN_WORKLOADS = {
    "llama70b_attn_prefill_tp8": AttnWorkload("llama70b_attn_prefill_tp8", 4096, 8192, 64, 8, 128,
                                              8, "Llama-70B attention projections, TP=8, prefill"),
    "llama70b_attn_decode_tp8": AttnWorkload("llama70b_attn_decode_tp8", 64, 8192, 64, 8, 128, 8,
                                             "Llama-70B attention projections, TP=8, decode",
                                             Ts=(1, 8, 64)),
    "gpt_attn_p4": AttnWorkload("gpt_attn_p4", 2048, 4096, 32, 32, 128, 4,
                                "GPT-style attention projections, 32 heads, p=4"),
}


def gaussian_f32(shape, seed: int, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) fp32 array from numpy's default_rng(seed)."""
    a = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def gaussian_bf16(shape, seed: int, std: float = 1.0):
    """N(0, std^2) drawn in fp32, rounded to bf16 (RNE) by torch; a CPU torch tensor."""
    import torch

    return torch.from_numpy(gaussian_f32(shape, seed, std)).to(torch.bfloat16)


def tiny_f32_inputs():
    """The Day 41 post's check: legacy RandomState(42), drawn in the order x, W, b (all
    N(0,1) fp32), then a down-projection W2 [2048, 512] ~ N(0,1)/sqrt(2048)."""
    rs = np.random.RandomState(42)
    X = rs.randn(4, 512).astype(np.float32)
    W1 = rs.randn(512, 2048).astype(np.float32)
    b1 = rs.randn(2048).astype(np.float32)
    W2 = (rs.randn(2048, 512) / np.sqrt(2048.0)).astype(np.float32)
    return X, W1, b1, W2


def gpt_gelu_shard_inputs(T: int = 2048, d: int = 4096, s: int = 4096):
    """Compact shard of the GPT-style GeLU MLP: X seed 42, W1_i seed 43, W2_i seed 44
    (bf16), b1_i = 0.  W1_i is [d, s], W2_i is [s, d]."""
    import torch

    X = gaussian_bf16((T, d), 42)
    W1 = gaussian_bf16((d, s), 43, WEIGHT_STD)
    W2 = gaussian_bf16((s, d), 44, WEIGHT_STD)
    b1 = torch.zeros(s, dtype=torch.bfloat16)
    return X, W1, b1, W2


def llama_shard_weights(d: int = 8192, s: int = 3584):
    """Compact TP=8 Llama-70B weight shard: W_gate seed 43, W_up seed 44 ([d, s]),
    W_down seed 45 ([s, d]); bf16 N(0, 0.02^2)."""
    Wg = gaussian_bf16((d, s), 43, WEIGHT_STD)
    Wu = gaussian_bf16((d, s), 44, WEIGHT_STD)
    W2 = gaussian_bf16((s, d), 45, WEIGHT_STD)
    return Wg, Wu, W2


def llama_tokens(T: int, d: int = 8192):
    """X [T, d] bf16 from seed 42; a smaller T gives the first rows of a larger draw."""
    return gaussian_bf16((T, d), 42)


def llama_full_weights(d: int = 8192, k: int = 28672):
    """Full (unsharded) Llama-70B MLP weights: Wg, Wu [d, k] seeds 43, 44; W2 [k, d] seed 45."""
    Wg = gaussian_bf16((d, k), 43, WEIGHT_STD)
    Wu = gaussian_bf16((d, k), 44, WEIGHT_STD)
    W2 = gaussian_bf16((k, d), 45, WEIGHT_STD)
    return Wg, Wu, W2


def small_case(T: int, d: int, k: int, seed: int, swiglu: bool, bias: bool, x_std: float = 1.0,
               w_std: float = WEIGHT_STD):
    """Generic small bf16 case: X, W1 (gate), Wu (or None), b1 (or None), W2 (full matrices)."""
    X = gaussian_bf16((T, d), seed, x_std)
    W1 = gaussian_bf16((d, k), seed + 1, w_std)
    Wu = gaussian_bf16((d, k), seed + 2, w_std) if swiglu else None
    b1 = gaussian_bf16((k,), seed + 3, 0.5) if bias else None
    W2 = gaussian_bf16((k, d), seed + 4, w_std)
    return X, W1, Wu, b1, W2


def attn_weights(d: int, Hq: int, Hkv: int, dh: int, seed: int = 46):
    """Full attention projection weights, bf16 N(0, 0.02^2): the packed QKV matrix
    [d, (Hq + 2 Hkv) dh] (query heads, then key heads, then value heads) from seed
    `seed`, the output projection [Hq dh, d] from seed + 1."""
    Wqkv = gaussian_bf16((d, (Hq + 2 * Hkv) * dh), seed, WEIGHT_STD)
    WO = gaussian_bf16((Hq * dh, d), seed + 1, WEIGHT_STD)
    return Wqkv, WO


def attn_output(T: int, width: int, seed: int = 48):
    """A stand-in for one shard's attention output [T, width], bf16 N(0, 1): the
    input of the row-parallel output projection."""
    return gaussian_bf16((T, width), seed)


def layernorm_params(d: int, seed: int, std: float = 0.1):
    """LayerNorm scale and shift [d], fp32 CPU tensors: 1 + N(0, std^2) from seed, and
    N(0, std^2) from seed + 1."""
    import torch

    g = 1.0 + gaussian_f32((d,), seed, std)
    b = gaussian_f32((d,), seed + 1, std)
    return torch.from_numpy(g.astype(np.float32)), torch.from_numpy(b)


def block_case(T: int, d: int, Hq: int, Hkv: int, dh: int, k: int, act: str, seed: int,
               bias: bool = True, full_weights: bool = False):
    """Inputs of one pre-LayerNorm transformer block (CPU tensors): the residual stream
    X [T, d] fp32 N(0, 1); the two LayerNorms' (scale, shift); the packed QKV weight
    [d, (Hq + 2 Hkv) dh] and the output projection [Hq dh, d]; the FFN weights W1 (gate)
    and Wu [d, k] (Wu for SwiGLU only) and W2 [k, d]; weights bf16 N(0, 0.02^2).
    Biases (if `bias`): bqkv and b1 bf16 N(0, 0.02^2), bO and b2 fp32 N(0, 0.02^2) (no
    b1 with SwiGLU).  With full_weights the weights are the Llama-70B draws (attention
    seeds 46/47, FFN seeds 43-45) instead of seed-derived ones."""
    import torch

    X = torch.from_numpy(gaussian_f32((T, d), seed))
    if full_weights:
        Wqkv, WO = attn_weights(d, Hq, Hkv, dh)
        W1, Wu, W2 = llama_full_weights(d, k)
        Wu = Wu if act == "swiglu" else None
    else:
        Wqkv, WO = attn_weights(d, Hq, Hkv, dh, seed + 1)
        W1 = gaussian_bf16((d, k), seed + 3, WEIGHT_STD)
        Wu = gaussian_bf16((d, k), seed + 4, WEIGHT_STD) if act == "swiglu" else None
        W2 = gaussian_bf16((k, d), seed + 5, WEIGHT_STD)
    case = dict(X=X, ln1=layernorm_params(d, seed + 6), ln2=layernorm_params(d, seed + 8),
                Wqkv=Wqkv, WO=WO, W1=W1, Wu=Wu, W2=W2)
    if bias:
        case["bqkv"] = gaussian_bf16(((Hq + 2 * Hkv) * dh,), seed + 10, WEIGHT_STD)
        case["bO"] = torch.from_numpy(gaussian_f32((d,), seed + 11, WEIGHT_STD))
        case["b2"] = torch.from_numpy(gaussian_f32((d,), seed + 12, WEIGHT_STD))
        if act != "swiglu":
            case["b1"] = gaussian_bf16((k,), seed + 13, WEIGHT_STD)
    return case


def attn_scaled(T: int, Hq: int, Hkv: int, dh: int, seed: int, score_std: float):
    """Q, K, V for the attention core with scores of a chosen spread: Q and K
    N(0, score_std) (so that q.k / sqrt(dh) has standard deviation score_std), V
    N(0, 1); bf16 CPU tensors from seeds seed, seed + 1, seed + 2."""
    a = float(np.sqrt(score_std))
    return (gaussian_bf16((T, Hq * dh), seed, a), gaussian_bf16((T, Hkv * dh), seed + 1, a),
            gaussian_bf16((T, Hkv * dh), seed + 2))


def attn_ramp(nseq: int, S: int, Hq: int, Hkv: int, dh: int, seed: int, slope: float):
    """Q, K, V whose scores move steadily along each sequence: every query is
    1 + N(0, 1) in each head dimension, key j of a sequence is slope * j +
    N(0, 0.25) in each, so the score of key j grows (slope > 0) or falls
    (slope < 0) by about sqrt(dh) * slope per key.  V N(0, 1).  bf16 CPU
    tensors (seeds seed, seed + 1, seed + 2)."""
    import torch

    T = nseq * S
    q = 1.0 + gaussian_f32((T, Hq * dh), seed)
    pos = np.tile(np.arange(S, dtype=np.float32), nseq)[:, None]
    k = np.float32(slope) * pos + gaussian_f32((T, Hkv * dh), seed + 1, 0.5)
    return (torch.from_numpy(q).to(torch.bfloat16), torch.from_numpy(k).to(torch.bfloat16),
            gaussian_bf16((T, Hkv * dh), seed + 2))


def attn_dominant(nseq: int, S: int, Hq: int, Hkv: int, dh: int, seed: int, causal: bool,
                  gain: float = 3.0):
    """Q, K, V in which every query has one key far above the others: K and V
    N(0, 1); query t of head h is gain times the key row of a key j*(t, h) drawn
    uniformly from the keys it sees (j* <= t under the causal mask), plus
    N(0, 0.1^2).  Its score with j* is about gain * sqrt(dh), the others about
    N(0, gain^2).  Returns the bf16 CPU tensors and j* [T, Hq] (positions within
    the sequence)."""
    import torch

    T = nseq * S
    grp = Hq // Hkv
    K = gaussian_f32((T, Hkv * dh), seed + 1)
    rng = np.random.default_rng(seed)
    t_in = np.tile(np.arange(S), nseq)
    hi = (t_in + 1) if causal else np.full(T, S)
    jstar = np.floor(rng.random((T, Hq)) * hi[:, None]).astype(np.int64)
    q = gaussian_f32((T, Hq * dh), seed + 3, 0.1)
    base = (np.arange(T) // S) * S
    for h in range(Hq):
        c = h // grp
        q[:, h * dh:(h + 1) * dh] += np.float32(gain) * K[base + jstar[:, h], c * dh:(c + 1) * dh]
    return (torch.from_numpy(q).to(torch.bfloat16), torch.from_numpy(K).to(torch.bfloat16),
            gaussian_bf16((T, Hkv * dh), seed + 2), jstar)
