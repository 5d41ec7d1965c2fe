"""The split-K paths under HIP-graph capture: a captured call is replayed
several times, with other eager calls that share the workspace (and leave its
arrival counters zero) and torch work in between, and every replay must give
the bits of the eager call.  The kernels clear their own counters; nothing in
the captured work is a memset."""
import pytest
import torch

import megatron_tensor_mlp_amd as tp
from megatron_tensor_mlp_amd import synth
from tests.helpers import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REPLAYS = 3


def dev(t):
    return None if t is None else t.to(DEV)


def mlp_case(ws, T, d, k, p, act, seed):
    sw = act == "swiglu"
    X, W1, Wu, b1, W2 = synth.small_case(T, d, k, seed, sw, bias=not sw)
    X, W1, Wu, b1, W2 = (dev(t) for t in (X, W1, Wu, b1, W2))
    Y = torch.empty(T, k // p, dtype=torch.bfloat16, device=DEV)
    Z = torch.empty(T, d, device=DEV)
    assert 0 < tp.tp_workspace_bytes(torch.bfloat16, act, T, d, k, p) <= ws.numel()

    def call():
        tp.tp_mlp_shard(X, W1, W2, p - 1, p, Y, Z, act=act, Wu=Wu, b1=b1, ws=ws)
    return call, (Y, Z)


def qkv_case(ws, T, d, Hq, Hkv, dh, seed):
    X = dev(synth.gaussian_bf16((T, d), seed))
    W = dev(synth.gaussian_bf16((d, (Hq + 2 * Hkv) * dh), seed + 1, synth.WEIGHT_STD))
    b = dev(synth.gaussian_bf16(((Hq + 2 * Hkv) * dh,), seed + 2, 0.5))
    out = torch.empty(T, (Hq + 2 * Hkv) * dh, dtype=torch.bfloat16, device=DEV)
    assert 0 < tp.tp_qkv_workspace_bytes(torch.bfloat16, T, d, Hq, Hkv, dh, 1) <= ws.numel()

    def call():
        tp.tp_qkv_linear(X, W, Hq, Hkv, dh, 0, 1, out, bqkv=b, ws=ws)
    return call, (out,)


CASES = {
    "tiled split-K (column 4 ranges, row 3)": lambda ws: mlp_case(ws, 300, 8192, 3584, 1, "swiglu", 41),
    "tiled split-K QKV (8 ranges)": lambda ws: qkv_case(ws, 1000, 8192, 8, 1, 128, 42),
    "few-token split-K (T = 8)": lambda ws: mlp_case(ws, 8, 1032, 4096, 2, "swiglu", 43),
    "few-token split-K (T = 64, GeLU)": lambda ws: mlp_case(ws, 64, 1032, 4096, 2, "gelu_tanh", 44),
}


@pytest.mark.parametrize("what", list(CASES))
def test_graph_replays_match_eager(what):
    say(f"graph case: {what}")
    ws = torch.zeros(96 << 20, dtype=torch.uint8, device=DEV)
    call, outs = CASES[what](ws)
    # another split-K call of a different shape on the same workspace, run
    # eagerly between replays
    other, _ = mlp_case(ws, 65, 12296, 1024, 4, "none", 45)
    call()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    assert int(ws[:256 << 10].count_nonzero()) == 0

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            call()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()

    for r in range(REPLAYS):
        for o in outs:
            o.fill_(float("nan"))
        # eager work between replays: torch ops and a library call on the
        # same workspace (its counters must come back to zero too)
        if r % 2 == 0:
            other()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, ref):
            assert torch.equal(o, e), f"replay {r} differs from the eager call"
        assert int(ws[:256 << 10].count_nonzero()) == 0
