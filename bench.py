"""Benchmark of one MI355X's tensor-parallel MLP shard.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--quick]

A step is one forward of one GPU's shard of the Llama-70B SwiGLU MLP at TP = 8
(T = 4096 tokens, d = 8192, k/p = 3584): the column step (X Wg_i, X Wu_i,
SiLU(g) * u -> bf16 Y_i) then the row step (Y_i W2_i -> fp32 partial Z_i),
i.e. the two launches tp_mlp_shard makes.  Inputs are seeded synthetic bf16
tensors already resident in HBM.  The timed region is bracketed by HIP events
on the launch stream; the headline GEMMs' per-launch durations are the
medians over 50 further steps with an event after each launch (the steady
state of the timed steps); the secondary sections time HIP-graph replays
(events only at the ends of a batch of launches).

Prints ONE JSON line.  `value` is the step's algorithmic TFLOP/s (2*T*d*(k/p)
flops per GEMM, three GEMMs).  Secondary fields report the few-token (decode)
shard in GB/s of weights streamed, the on-device partial sum in GB/s, the
simulated TP = 8 block, the GPT-style GeLU shard, the attention projections
of one head shard (QKV and output projection) and the shard's training step
(forward that keeps the pre-activation, and the backward pass), and the MFMA
and HBM calibrations, and the vendor GEMM (hipBLASLt through torch.matmul) on
the headline's shapes for comparison.  `roofline` covers the dominant kernel
(the SwiGLU column GEMM), `roofline_decode` and `roofline_partial_sum` the
HBM-bound steps;
`cpu_baseline` is the CPU oracle timed on a bounded row sample of the same
workload, and (`configs`) on a sample of every other configuration next to the
GPU path's errors against it there.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("MLP-shard TFLOP/s & % bf16 MFMA peak (prefill); GB/s & % HBM peak (decode)")
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")
TILED_SOURCES = ["megatron_tensor_mlp_amd/csrc/gemm_tiled.hip",
                 "megatron_tensor_mlp_amd/csrc/tiled_geometry.hpp",
                 "megatron_tensor_mlp_amd/csrc/lds_dma.hpp",
                 "megatron_tensor_mlp_amd/csrc/device_common.hpp",
                 "megatron_tensor_mlp_amd/csrc/kernels.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel_tag):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel source (else None)."""
    path = os.path.join(PROFILES, f"{kernel_tag}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    h = re.search(r"source_sha256_16:\s*([0-9a-f]+)", text)
    if not m or not h or h.group(1) != source_hash(TILED_SOURCES):
        return None
    return float(m.group(1))


def time_graph(torch, fn_list, steps, warmup, per_replay=5):
    """Capture `per_replay` rounds of the launches in fn_list into one HIP graph
    and time `steps` replays (after `warmup`): GPU time per round, without
    host launch gaps.  Every launch is run once eagerly first so nothing is
    allocated during capture."""
    for fn in fn_list:
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            for _ in range(per_replay):
                for fn in fn_list:
                    fn()
    torch.cuda.synchronize()
    for _ in range(max(1, warmup)):
        graph.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for r in range(steps):
        graph.replay()
        ev[r + 1].record()
    torch.cuda.synchronize()
    per = [ev[r].elapsed_time(ev[r + 1]) / 1e3 / per_replay for r in range(steps)]
    global LAST_SPREAD
    LAST_SPREAD = spread(per)
    return ev[0].elapsed_time(ev[steps]) / 1e3 / (steps * per_replay)


LAST_SPREAD = None


def spread(times):
    """Median, p10 and p90 of per-iteration times (seconds), in microseconds."""
    t = sorted(times)
    q = lambda f: t[min(len(t) - 1, int(round(f * (len(t) - 1))))]  # noqa: E731
    return {"median_us": round(q(0.5) * 1e6, 2), "p10_us": round(q(0.1) * 1e6, 2),
            "p90_us": round(q(0.9) * 1e6, 2), "iterations": len(t)}


def time_each(torch, fn_list, n, warmup):
    """Per-iteration times of n rounds of the launches in fn_list (after
    `warmup`), with an event pair around every round on the current stream."""
    for _ in range(warmup):
        for fn in fn_list:
            fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    ev[0].record()
    for r in range(n):
        for fn in fn_list:
            fn()
        ev[r + 1].record()
    torch.cuda.synchronize()
    return [ev[r].elapsed_time(ev[r + 1]) / 1e3 for r in range(n)]


def time_legs(torch, fn_list, n, warmup):
    """Per-launch durations inside n steps of the launches in fn_list: an event
    on the launch stream before the first launch of a step and after each
    launch, so the legs of a step add up to the step.  Returns one list of n
    durations (seconds) per launch, and the n step durations."""
    for _ in range(warmup):
        for fn in fn_list:
            fn()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fn_list) + 1)]
          for _ in range(n)]
    for r in range(n):
        ev[r][0].record()
        for j, fn in enumerate(fn_list):
            fn()
            ev[r][j + 1].record()
    torch.cuda.synchronize()
    legs = [[ev[r][j].elapsed_time(ev[r][j + 1]) / 1e3 for r in range(n)]
            for j in range(len(fn_list))]
    steps = [ev[r][0].elapsed_time(ev[r][-1]) / 1e3 for r in range(n)]
    return legs, steps


def median(xs):
    t = sorted(xs)
    return t[len(t) // 2]


def time_steps(torch, fn_list, steps, warmup):
    """Wall time of `steps` rounds of the launches in fn_list (after `warmup`),
    bracketed by a synchronisation and an event pair on the current stream."""
    for _ in range(warmup):
        for fn in fn_list:
            fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        for fn in fn_list:
            fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3


RAMP_S = 0.15


def ramp(torch, fn_list, seconds=RAMP_S):
    """Run rounds of fn_list for `seconds` of wall time.  After idling, the GPU
    starts a sustained MFMA load at a low clock and needs ~50 prefill steps
    (~35 ms) to reach its steady state (per-step time 850 -> 625 us); this
    runs before the warm-up so that the timed steps measure that state."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            for fn in fn_list:
                fn()
        torch.cuda.synchronize()


def headline(torch, tp, synth, steps, warmup):
    """The timed region: `steps` shard forwards back to back, after the clock
    ramp and `warmup` untimed steps.  Per-kernel durations are the medians
    over 50 more steps with an event on the launch stream after each launch,
    so the two legs of a step add up to the step."""
    W = synth.WORKLOADS["llama70b_prefill_tp8"]
    dev = "cuda:0"
    Wg, Wu, W2 = (t.to(dev) for t in synth.llama_shard_weights(W.d, W.s))
    X = synth.llama_tokens(W.T, W.d).to(dev)
    Y = torch.empty(W.T, W.s, dtype=torch.bfloat16, device=dev)
    Z = torch.empty(W.T, W.d, dtype=torch.float32, device=dev)
    col = lambda: tp.tp_col_linear(X, Wg, 0, 1, Y, act="swiglu", Wu=Wu)  # noqa: E731
    row = lambda: tp.tp_row_linear(Y, W2, 0, 1, Z)  # noqa: E731
    ramp(torch, [col, row])
    total = time_steps(torch, [col, row], steps, warmup)
    # The same steps again, with an event after each launch: the per-kernel
    # durations of the steady state the timed steps ran in.
    legs, steps_ev = time_legs(torch, [col, row], 50, 0)
    flops_col = 2.0 * W.T * W.d * W.s * 2
    flops_row = 2.0 * W.T * W.d * W.s
    return dict(W=W, total=total, t_col=median(legs[0]), t_row=median(legs[1]),
                step_spread=spread(steps_ev), col_spread=spread(legs[0]),
                row_spread=spread(legs[1]), flops_col=flops_col, flops_row=flops_row,
                step_flops=flops_col + flops_row)


def decode_bench(torch, tp, synth, steps, warmup, rotate_bytes=600 << 20):
    """Few-token shard (column step then row step, the launches tp_mlp_shard
    makes).  Weights rotate over enough copies that every timed sequence
    touches more than 2x the 256 MB Infinity Cache before it comes back to a
    copy (the step: 4 x 176 MB; the column step alone: 6 x 117 MB; the row
    step alone: 11 x 59 MB), so they are read from HBM.  Timed by HIP-graph
    replay: a decode step is ~20-50 us of GPU work, where host launch gaps
    would otherwise count."""
    W = synth.WORKLOADS["llama70b_decode_tp8"]
    dev = "cuda:0"
    base = [t.to(dev) for t in synth.llama_shard_weights(W.d, W.s)]
    col_bytes = 2 * W.d * W.s * 2
    row_bytes = W.s * W.d * 2
    ncol = -(-rotate_bytes // col_bytes)
    nrow = -(-rotate_bytes // row_bytes)
    copies = -(-rotate_bytes // (col_bytes + row_bytes))
    sets = [base] + [[t.clone() for t in base] for _ in range(max(ncol, nrow) - 1)]
    out = {}
    wbytes = sum(t.numel() * t.element_size() for t in base)
    for T in W.Ts:
        X = synth.llama_tokens(T, W.d).to(dev)
        Y = torch.empty(T, W.s, dtype=torch.bfloat16, device=dev)
        Z = torch.empty(T, W.d, dtype=torch.float32, device=dev)
        ws = tp.workspace(tp.tp_workspace_bytes(torch.bfloat16, "swiglu", T, W.d, W.s, 1), dev)
        cols, rows = [], []
        for (Wg, Wu, W2) in sets:
            cols.append(lambda Wg=Wg, Wu=Wu: tp.tp_col_linear(X, Wg, 0, 1, Y, act="swiglu", Wu=Wu,
                                                               ws=ws))
            rows.append(lambda W2=W2: tp.tp_row_linear(Y, W2, 0, 1, Z, ws=ws))
        both = [f for pair in zip(cols[:copies], rows[:copies]) for f in pair]
        step = time_graph(torch, both, max(steps, 20), warmup) / copies
        step_spread = {k: (round(v / copies, 2) if k.endswith("_us") else v)
                       for k, v in LAST_SPREAD.items()}
        t_col = time_graph(torch, cols[:ncol], steps, warmup) / ncol
        t_row = time_graph(torch, rows[:nrow], steps, warmup) / nrow
        alg_bytes = wbytes + T * W.d * 2 + 2 * T * W.s * 2 + T * W.d * 4
        out[f"T{T}"] = {
            "us_per_step": round(step * 1e6, 2),
            "GBps": round(alg_bytes / step / 1e9, 1),
            "frac_hbm": round(alg_bytes / step / 1e9 / PEAK_HBM_GBS, 4),
            "alg_bytes": alg_bytes,
            "step_spread": step_spread,
            "col_us": round(t_col * 1e6, 2), "row_us": round(t_row * 1e6, 2),
            "col_GBps": round((2 * W.d * W.s * 2) / t_col / 1e9, 1),
            "row_GBps": round((W.s * W.d * 2) / t_row / 1e9, 1),
        }
    out["weight_bytes"] = wbytes
    out["rotation_copies"] = {"step": copies, "col": ncol, "row": nrow}
    out["timing"] = "HIP graph replay"
    return out


def partial_sum_bench(torch, tp, steps, warmup, copies=4):
    """The simulated TP=8 block's reduction: 8 fp32 [512, 8192] partials -> Z,
    rotating over `copies` sets (4 x 151 MB, more than twice the 256 MB
    Infinity Cache); HIP-graph replay."""
    dev = "cuda:0"
    p, T, d = 8, 512, 8192
    bufs = [torch.randn(p, T, d, device=dev) for _ in range(copies)]
    Zs = [torch.empty(T, d, device=dev) for _ in range(copies)]
    fns = [lambda b=b, z=z: tp.tp_partial_sum([b[q] for q in range(p)], z) for b, z in
           zip(bufs, Zs)]
    t = time_graph(torch, fns, max(20, steps), warmup) / copies
    sp = {k: (round(v / copies, 2) if k.endswith("_us") else v) for k, v in LAST_SPREAD.items()}
    nbytes = (p + 1) * T * d * 4
    return {"us": round(t * 1e6, 2), "GBps": round(nbytes / t / 1e9, 1),
            "frac_hbm": round(nbytes / t / 1e9 / PEAK_HBM_GBS, 4), "bytes": nbytes,
            "spread": sp, "rotation_copies": copies, "timing": "HIP graph replay"}


def hbm_calibration(torch, tp, steps, warmup, rotate_bytes=600 << 20):
    """Per-launch streaming-read rate of a plain read kernel (tp_calib_hbm_read)
    at the sizes the few-token kernels stream (the column step's 117 MB of gate
    and up weights, the row step's 59 MB) and at 2 GiB, buffers rotating past
    the Infinity Cache: the ceiling a single launch of that size reaches, ramp
    and drain included."""
    dev = "cuda:0"
    nwg = 1024
    sink = torch.zeros(nwg, dtype=torch.int32, device=dev)
    out = {}
    for name, nbytes in (("col_117MB", 2 * 8192 * 3584 * 2), ("row_59MB", 3584 * 8192 * 2),
                         ("2GiB", 2 << 30)):
        copies = max(1, -(-rotate_bytes // nbytes))
        bufs = [torch.ones(nbytes // 4, dtype=torch.int32, device=dev) for _ in range(copies)]
        fns = [lambda b=b: tp.tp_calib_hbm_read(b, sink) for b in bufs]
        t = time_graph(torch, fns, max(10, steps), warmup, per_replay=2) / copies
        out[name] = {"bytes": nbytes, "us": round(t * 1e6, 2), "GBps": round(nbytes / t / 1e9, 1),
                     "frac_hbm": round(nbytes / t / 1e9 / PEAK_HBM_GBS, 4),
                     "rotation_copies": copies}
        del bufs, fns
    out["kernel"] = ("tp_calib_hbm_read: 1024 workgroups x 256 threads, each a contiguous "
                     "1/1024 of the buffer, 16-byte nontemporal loads, 8 in flight per thread; "
                     "HIP-graph replay")
    return out


def simulated_block_bench(torch, tp, synth, steps, warmup):
    W = synth.WORKLOADS["llama70b_block_sim_tp8"]
    dev = "cuda:0"
    Wg, Wu, W2 = (t.to(dev) for t in synth.llama_full_weights(W.d, W.k))
    X = synth.llama_tokens(W.T, W.d).to(dev)
    Y = torch.empty(W.p, W.T, W.s, dtype=torch.bfloat16, device=dev)
    Zp = torch.empty(W.p, W.T, W.d, device=dev)
    Z = torch.empty(W.T, W.d, device=dev)
    fn = lambda: tp.tp_mlp_simulated(X, Wg, W2, W.p, Y, Zp, Z, act="swiglu", Wu=Wu)  # noqa: E731
    ramp(torch, [fn])
    t = time_graph(torch, [fn], max(10, steps), warmup, per_replay=2)
    sp = LAST_SPREAD
    flops = 2.0 * W.T * W.d * W.k * 3
    return {"us": round(t * 1e6, 1), "TFLOPs": round(flops / t / 1e12, 1),
            "frac_mfma": round(flops / t / 1e12 / PEAK_BF16_TFLOPS, 4), "spread": sp}


def gpt_bench(torch, tp, synth, steps, warmup):
    W = synth.WORKLOADS["gpt_gelu_p4"]
    dev = "cuda:0"
    X, W1, b1, W2 = (t.to(dev) for t in synth.gpt_gelu_shard_inputs(W.T, W.d, W.s))
    Y = torch.empty(W.T, W.s, dtype=torch.bfloat16, device=dev)
    Z = torch.empty(W.T, W.d, device=dev)
    col = lambda: tp.tp_col_linear(X, W1, 0, 1, Y, act="gelu_tanh", b1=b1)  # noqa: E731
    row = lambda: tp.tp_row_linear(Y, W2, 0, 1, Z)  # noqa: E731
    ramp(torch, [col, row])
    t = time_graph(torch, [col, row], max(20, steps), warmup)
    sp = LAST_SPREAD
    tc = time_graph(torch, [col], max(1, steps), warmup)
    tr = time_graph(torch, [row], max(1, steps), warmup)
    flops = 2.0 * W.T * W.d * W.s * 2
    return {"us": round(t * 1e6, 1), "TFLOPs": round(flops / t / 1e12, 1),
            "frac_mfma": round(flops / t / 1e12 / PEAK_BF16_TFLOPS, 4), "spread": sp,
            "col_us": round(tc * 1e6, 1), "row_us": round(tr * 1e6, 1)}


def attention_bench(torch, tp, synth, steps, warmup, rotate_bytes=600 << 20):
    """Attention block of one head shard of Llama-70B at TP = 8 (64 query and 8
    key/value heads of 128, d = 8192): the fused QKV projection (tp_qkv_linear,
    shard 3 of the full packed weight), the causal attention core (tp_attention,
    8 query heads on 1 key/value head) and the output projection's row block
    (tp_row_linear; timed alone on a stand-in attention output).
    Prefill T = 4096 after the clock ramp; decode T = 1, 8, 64 with the weights
    rotating over the 8 shards of 2 copies of the full matrices (16 x 38 MB, more
    than twice the 256 MB Infinity Cache).  HIP-graph replay."""
    W = synth.ATTN_WORKLOADS["llama70b_attn_prefill_tp8"]
    dev = "cuda:0"
    Wqkv, WO = (t.to(dev) for t in synth.attn_weights(W.d, W.Hq, W.Hkv, W.dh))
    out = {}
    X = synth.llama_tokens(W.T, W.d).to(dev)
    QKV = torch.empty(W.T, W.qkv_cols, dtype=torch.bfloat16, device=dev)
    O = synth.attn_output(W.T, W.o_rows).to(dev)
    Z = torch.empty(W.T, W.d, device=dev)
    qkv = lambda: tp.tp_qkv_linear(X, Wqkv, W.Hq, W.Hkv, W.dh, 3, W.p, QKV)  # noqa: E731
    row = lambda: tp.tp_row_linear(O, WO, 3, W.p, Z)  # noqa: E731
    hq, hkv = W.Hq // W.p, W.Hkv // W.p
    qw, kw = hq * W.dh, hkv * W.dh
    Oc = torch.empty(W.T, W.o_rows, dtype=torch.bfloat16, device=dev)
    core = lambda: tp.tp_attention(QKV[:, :qw], QKV[:, qw:qw + kw], QKV[:, qw + kw:], Oc,  # noqa
                                   hq, hkv, W.dh)
    blockf = lambda: tp.tp_row_linear(Oc, WO, 3, W.p, Z)  # noqa: E731
    ramp(torch, [qkv, row])
    t = time_graph(torch, [qkv, row], max(10, steps), warmup)
    sp = LAST_SPREAD
    tq = time_graph(torch, [qkv], max(5, steps), warmup)
    tr = time_graph(torch, [row], max(5, steps), warmup)
    tc = time_graph(torch, [core], max(5, steps), warmup)
    tb = time_graph(torch, [qkv, core, blockf], max(5, steps), warmup)
    fq = 2.0 * W.T * W.d * W.qkv_cols
    fr = 2.0 * W.T * W.o_rows * W.d
    fc = 4.0 * W.dh * hq * (W.T * (W.T + 1) / 2)  # causal: query t sees t + 1 keys
    out["prefill"] = {
        "workload": W.name, "T": W.T, "us": round(t * 1e6, 1),
        "TFLOPs": round((fq + fr) / t / 1e12, 1),
        "frac_mfma": round((fq + fr) / t / 1e12 / PEAK_BF16_TFLOPS, 4), "spread": sp,
        "qkv_us": round(tq * 1e6, 1), "qkv_TFLOPs": round(fq / tq / 1e12, 1),
        "o_proj_us": round(tr * 1e6, 1), "o_proj_TFLOPs": round(fr / tr / 1e12, 1),
        "core_us": round(tc * 1e6, 1), "core_TFLOPs": round(fc / tc / 1e12, 1),
        "core_flops": fc, "block_us": round(tb * 1e6, 1),
        "block_TFLOPs": round((fq + fr + fc) / tb / 1e12, 1)}
    del X, QKV, O, Z, Oc
    Wd = synth.ATTN_WORKLOADS["llama70b_attn_decode_tp8"]
    sets = [(Wqkv, WO), (Wqkv.clone(), WO.clone())]
    pairs = [(s, i) for s in sets for i in range(W.p)]
    wbytes = W.weight_bytes()
    dec = {}
    for T in Wd.Ts:
        X = synth.llama_tokens(T, W.d).to(dev)
        QKV = torch.empty(T, W.qkv_cols, dtype=torch.bfloat16, device=dev)
        O = synth.attn_output(T, W.o_rows).to(dev)
        Z = torch.empty(T, W.d, device=dev)
        ws = tp.workspace(max(tp.tp_qkv_workspace_bytes(torch.bfloat16, T, W.d, W.Hq, W.Hkv, W.dh,
                                                        W.p),
                              tp.tp_workspace_bytes(torch.bfloat16, "none", T, W.d, W.Hq * W.dh,
                                                    W.p)), dev)
        fns = []
        for (wq, wo), i in pairs:
            fns.append(lambda wq=wq, i=i: tp.tp_qkv_linear(X, wq, W.Hq, W.Hkv, W.dh, i, W.p, QKV,
                                                            ws=ws))
            fns.append(lambda wo=wo, i=i: tp.tp_row_linear(O, wo, i, W.p, Z, ws=ws))
        t = time_graph(torch, fns, max(steps, 20), warmup) / len(pairs)
        sp = {k: (round(v / len(pairs), 2) if k.endswith("_us") else v)
              for k, v in LAST_SPREAD.items()}
        tq = time_graph(torch, fns[0::2], max(steps, 20), warmup) / len(pairs)
        alg = wbytes + T * W.d * 2 + T * W.qkv_cols * 2 + T * W.o_rows * 2 + T * W.d * 4
        dec[f"T{T}"] = {"us_per_step": round(t * 1e6, 2), "GBps": round(alg / t / 1e9, 1),
                        "frac_hbm": round(alg / t / 1e9 / PEAK_HBM_GBS, 4), "step_spread": sp,
                        "qkv_us": round(tq * 1e6, 2),
                        "qkv_GBps": round(2 * W.d * W.qkv_cols / tq / 1e9, 1)}
    dec["weight_bytes"] = wbytes
    dec["rotation"] = "8 shards x 2 copies"
    out["decode"] = dec
    out["timing"] = "HIP graph replay"
    return out


def transformer_block_bench(torch, tp, synth, steps, warmup):
    """One pre-LayerNorm Llama-70B transformer block (d = 8192, 64 query and 8
    key/value heads of 128, SwiGLU FFN k = 28672) of 8 tensor-parallel shards
    simulated on this GPU (tp_block_simulated, full weights): prefill, one
    causal sequence of 4096 tokens, and decode, one token.  The row steps
    (tp_residual_layernorm) are timed alone as well: LN1 of the residual stream,
    and the sum of the 8 partials with the bias and the residual followed by LN2.
    HIP-graph replay."""
    dev = "cuda:0"
    d, Hq, Hkv, dh, k, p = 8192, 64, 8, 128, 28672, 8
    ncol = (Hq + 2 * Hkv) * dh
    out = {"workload": "llama70b_block_tp8 (8 shards simulated)"}
    c = None
    for T in (4096, 1):
        c = synth.block_case(T, d, Hq, Hkv, dh, k, "swiglu", seed=42, full_weights=True) \
            if c is None else dict(c, X=torch.from_numpy(synth.gaussian_f32((T, d), 42)))
        g = {n: (tuple(x.to(dev) for x in v) if isinstance(v, tuple) else
                 (v.to(dev) if v is not None else None)) for n, v in c.items()}
        Out = torch.empty(T, d, device=dev)
        ws = tp.workspace(tp.tp_block_workspace_bytes(torch.bfloat16, "swiglu", 1, T, d, Hq, Hkv,
                                                      dh, k, p), dev)
        f = lambda T=T, g=g, Out=Out, ws=ws: tp.tp_block_simulated(  # noqa: E731
            g["X"], Hq, Hkv, dh, p, g["ln1"], g["Wqkv"], g["WO"], g["ln2"], g["W1"], g["W2"], Out,
            S=T, act="swiglu", bqkv=g["bqkv"], bO=g["bO"], Wu=g["Wu"], b2=g["b2"], ws=ws)
        ramp(torch, [f])
        t = time_graph(torch, [f], max(3, steps), warmup, per_replay=2)
        flops = (2.0 * T * d * ncol + 4.0 * dh * Hq * T * (T + 1) / 2 + 2.0 * T * Hq * dh * d
                 + 6.0 * T * d * k)
        wbytes = 2.0 * (d * ncol + Hq * dh * d + 3 * d * k)
        key = "prefill" if T > 1 else "decode"
        out[key] = {"T": T, "us": round(t * 1e6, 1), "TFLOPs": round(flops / t / 1e12, 1),
                    "frac_mfma": round(flops / t / 1e12 / PEAK_BF16_TFLOPS, 4),
                    "weight_GBps": round(wbytes / t / 1e9, 1), "flops": flops,
                    "weight_bytes": wbytes, "spread": LAST_SPREAD}
        if T > 1:
            Xr, Ab, X1 = g["X"], torch.empty(T, d, dtype=torch.bfloat16, device=dev), \
                torch.empty(T, d, device=dev)
            parts = [torch.empty(T, d, device=dev).normal_() for _ in range(p)]
            ln1 = lambda: tp.tp_residual_layernorm((), A=Ab, R=Xr, gamma=g["ln1"][0],  # noqa
                                                   beta=g["ln1"][1])
            red = lambda: tp.tp_residual_layernorm(parts, X=X1, A=Ab, bias=g["bO"], R=Xr,  # noqa
                                                   gamma=g["ln2"][0], beta=g["ln2"][1])
            t1 = time_graph(torch, [ln1], max(5, steps), warmup)
            t2 = time_graph(torch, [red], max(5, steps), warmup)
            b1 = T * d * (4 + 2)
            b2 = T * d * (4 * p + 4 + 4 + 2)
            out["row_steps"] = {
                "layernorm_us": round(t1 * 1e6, 1), "layernorm_GBps": round(b1 / t1 / 1e9, 1),
                "reduce8_residual_layernorm_us": round(t2 * 1e6, 1),
                "reduce8_residual_layernorm_GBps": round(b2 / t2 / 1e9, 1),
                "bytes": {"layernorm": b1, "reduce8_residual_layernorm": b2}}
            del parts, X1, Ab
        del g, Out
    out["timing"] = "HIP graph replay"
    return out


def backward_bench(torch, tp, synth, steps, warmup):
    """Training step of the Llama-70B SwiGLU shard at TP = 8, T = 4096: the
    training forward of the column step (Y and the kept [G | U]), the row step,
    and the shard backward (dH = dY * SwiGLU', the dX term, dWg, dWu, dW2) from
    a seeded dZ.  Algorithmic flops: 3 GEMMs forward, 6 backward, 2 T d (k/p)
    each.  HIP-graph replay after the clock ramp."""
    W = synth.WORKLOADS["llama70b_prefill_tp8"]
    dev = "cuda:0"
    T, d, s = W.T, W.d, W.s
    Wg, Wu, W2 = (t.to(dev) for t in synth.llama_shard_weights(d, s))
    X = synth.llama_tokens(T, d).to(dev)
    dZ = synth.gaussian_bf16((T, d), 46).to(dev)
    Y = torch.empty(T, s, dtype=torch.bfloat16, device=dev)
    H = torch.empty(T, 2 * s, dtype=torch.bfloat16, device=dev)
    Z = torch.empty(T, d, device=dev)
    dH = torch.empty(T, 2 * s, dtype=torch.bfloat16, device=dev)
    dXp = torch.empty(T, d, device=dev)
    dWg = torch.empty(d, s, device=dev)
    dWu = torch.empty(d, s, device=dev)
    dW2 = torch.empty(s, d, device=dev)
    fwd = [lambda: tp.tp_col_linear_train(X, Wg, 0, 1, Y, H, act="swiglu", Wu=Wu),
           lambda: tp.tp_row_linear(Y, W2, 0, 1, Z)]
    bwd = lambda: tp.tp_mlp_shard_backward(X, Wg, W2, H, Y, dZ, 0, 1, dH, dXp, dWg, dW2,  # noqa
                                           act="swiglu", Wu=Wu, dWu=dWu)
    ramp(torch, fwd + [bwd])
    tb = time_graph(torch, [bwd], max(5, steps), warmup, per_replay=2)
    sb = LAST_SPREAD
    tf = time_graph(torch, fwd, max(5, steps), warmup, per_replay=2)
    tt = time_graph(torch, fwd + [bwd], max(5, steps), warmup, per_replay=2)
    st = LAST_SPREAD
    unit = 2.0 * T * d * s
    return {"workload": W.name, "T": T,
            "backward_us": round(tb * 1e6, 1), "backward_TFLOPs": round(6 * unit / tb / 1e12, 1),
            "backward_frac_mfma": round(6 * unit / tb / 1e12 / PEAK_BF16_TFLOPS, 4),
            "backward_spread": sb,
            "train_forward_us": round(tf * 1e6, 1),
            "train_forward_TFLOPs": round(3 * unit / tf / 1e12, 1),
            "train_step_us": round(tt * 1e6, 1), "train_step_TFLOPs": round(9 * unit / tt / 1e12, 1),
            "train_step_spread": st, "flops_backward": 6 * unit, "timing": "HIP graph replay"}


def mfma_calibration(torch, tp, iters=20000, nwg=1024):
    """Sustained dense bf16 MFMA rate and the shader clock it runs at, for zero
    operands and for operands with the workloads' value mix (A ~ N(0,1),
    B ~ N(0, 0.02^2)).  The chip holds its power limit by lowering the clock,
    and random operands draw more power than zeros, so the second figure is
    the MFMA ceiling that applies to these workloads (the published peak
    assumes 2.4 GHz)."""
    dev = "cuda:0"
    out = {}
    flops = nwg * 4 * iters * 8 * 32768.0
    for name, gaussian in (("zeros", False), ("gaussian", True)):
        stats = torch.zeros(2 * nwg, dtype=torch.int64, device=dev)
        for _ in range(2):
            tp.tp_calib_mfma_bf16(gaussian, iters, stats)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        tp.tp_calib_mfma_bf16(gaussian, iters, stats)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / 1e3
        st = stats.cpu()
        ghz = float(st[0::2].sum()) / float(st[1::2].sum()) * 0.1
        tf = flops / t / 1e12
        out[name] = {"TFLOPs": round(tf, 1), "clock_GHz": round(ghz, 3),
                     "frac_published_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    out["kernel"] = "v_mfma_f32_32x32x16_bf16 loop, 1024 workgroups x 4 waves (tp_calib_mfma_bf16)"
    return out


def library_gemm_reference(torch, synth, steps, warmup):
    """The vendor GEMM (torch.matmul, i.e. hipBLASLt) on the headline's shapes,
    timed the same way as the shard's launches, as a check of the harness and
    a point of comparison only (it is not part of the path): the column step
    as one GEMM over the concatenated [Wg_i | Wu_i] (no SwiGLU epilogue, so
    it does less than the path's column launch) and the row step with a bf16
    output (half the output bytes of the path's fp32 partial)."""
    W = synth.WORKLOADS["llama70b_prefill_tp8"]
    dev = "cuda:0"
    Wg, Wu, W2 = (t.to(dev) for t in synth.llama_shard_weights(W.d, W.s))
    X = synth.llama_tokens(W.T, W.d).to(dev)
    Wgu = torch.cat([Wg, Wu], dim=1).contiguous()
    Y = torch.empty(W.T, W.s, dtype=torch.bfloat16, device=dev).normal_()
    G = torch.empty(W.T, 2 * W.s, dtype=torch.bfloat16, device=dev)
    Z = torch.empty(W.T, W.d, dtype=torch.bfloat16, device=dev)
    col = lambda: torch.matmul(X, Wgu, out=G)  # noqa: E731
    row = lambda: torch.matmul(Y, W2, out=Z)  # noqa: E731
    ramp(torch, [col, row])
    legs, _ = time_legs(torch, [col, row], max(20, steps), warmup)
    t_col, t_row = median(legs[0]), median(legs[1])
    f_col = 2.0 * W.T * W.d * 2 * W.s
    f_row = 2.0 * W.T * W.d * W.s
    return {"col_us": round(t_col * 1e6, 2), "col_TFLOPs": round(f_col / t_col / 1e12, 1),
            "row_bf16_out_us": round(t_row * 1e6, 2),
            "row_bf16_out_TFLOPs": round(f_row / t_row / 1e12, 1),
            "what": "torch.matmul (hipBLASLt) on X [4096, 8192] x [Wg_i | Wu_i] [8192, 7168] -> bf16, "
                    "and Y_i [4096, 3584] x W2_i [3584, 8192] -> bf16; events around each launch"}


def _errors(np, got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    d = got - ref
    return (float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300)),
            float(np.max(np.abs(d)) / max(np.max(np.abs(ref)), 1e-300)))


def oracle_configs(torch, tp, synth):
    """Every workload configuration: the oracle's wall time on a stated sample,
    and the GPU path's error against the oracle on that sample (relative
    Frobenius and largest error relative to the largest reference value)."""
    import numpy as np

    import oracle

    dev = "cuda:0"
    f = lambda t: t.detach().to("cpu").to(torch.float64).numpy()  # noqa: E731
    out = {}

    def entry(name, sample, dt, pairs, bar):
        e = {"sample": sample, "oracle_s": round(dt, 3), "bar": bar}
        for what, got, ref in pairs:
            fro, mx = _errors(np, got, ref)
            e[what] = {"rel_fro": float(f"{fro:.3e}"), "max_rel": float(f"{mx:.3e}")}
        out[name] = e

    # tiny fp32, p = 4 simulated: every output, against the unsharded oracle
    X, W1, b1, W2 = synth.tiny_f32_inputs()
    tt = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    Yd = torch.empty(4, 4, 512, device=dev)
    Zp = torch.empty(4, 4, 512, device=dev)
    Zd = torch.empty(4, 512, device=dev)
    tp.tp_mlp_simulated(tt(X), tt(W1), tt(W2), 4, Yd, Zp, Zd, act="gelu_tanh", b1=tt(b1))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    Zr = oracle.mlp_unsharded(X, W1, W2, "gelu_tanh", b1=b1)
    entry("tiny_f32_p4", "all 4 rows (unsharded oracle)", time.perf_counter() - t0,
          [("Z", f(Zd), Zr)], "rel_fro <= 1e-5")

    bf_bar = "rel_fro <= 5e-3 and max_rel <= 2e-2"
    # GPT-style GeLU shard, p = 4: the GPU computes every row, the oracle the first 32
    W = synth.WORKLOADS["gpt_gelu_p4"]
    X, W1, b1, W2 = synth.gpt_gelu_shard_inputs(W.T, W.d, W.s)
    Y = torch.empty(W.T, W.s, dtype=torch.bfloat16, device=dev)
    Z = torch.empty(W.T, W.d, device=dev)
    tp.tp_mlp_shard(X.to(dev), W1.to(dev), W2.to(dev), 0, 1, Y, Z, act="gelu_tanh",
                    b1=b1.to(dev))
    torch.cuda.synchronize()
    r = 32
    t0 = time.perf_counter()
    Yr, Zr = oracle.mlp_shard(f(X[:r]), f(W1), f(W2), 0, 1, "gelu_tanh", b1=f(b1))
    entry(W.name, f"first {r} of {W.T} token rows", time.perf_counter() - t0,
          [("Y", f(Y[:r]), Yr), ("Z", f(Z[:r]), Zr)], bf_bar)
    del Y, Z

    # Llama-70B prefill shard: every row on the GPU, the first 16 in the oracle
    W = synth.WORKLOADS["llama70b_prefill_tp8"]
    Wg, Wu, W2 = synth.llama_shard_weights(W.d, W.s)
    Wgd, Wud, W2d = Wg.to(dev), Wu.to(dev), W2.to(dev)
    Wg64, Wu64, W264 = f(Wg), f(Wu), f(W2)
    X = synth.llama_tokens(W.T, W.d)
    Y = torch.empty(W.T, W.s, dtype=torch.bfloat16, device=dev)
    Z = torch.empty(W.T, W.d, device=dev)
    tp.tp_mlp_shard(X.to(dev), Wgd, W2d, 0, 1, Y, Z, act="swiglu", Wu=Wud)
    torch.cuda.synchronize()
    r = 16
    t0 = time.perf_counter()
    Yr, Zr = oracle.mlp_shard(f(X[:r]), Wg64, W264, 0, 1, "swiglu", Wu=Wu64)
    entry(W.name, f"first {r} of {W.T} token rows", time.perf_counter() - t0,
          [("Y", f(Y[:r]), Yr), ("Z", f(Z[:r]), Zr)], bf_bar)
    del Y, Z

    # decode, T = 1, 8, 64: every row
    for T in synth.WORKLOADS["llama70b_decode_tp8"].Ts:
        Xt = synth.llama_tokens(T, W.d)
        Y = torch.empty(T, W.s, dtype=torch.bfloat16, device=dev)
        Z = torch.empty(T, W.d, device=dev)
        tp.tp_mlp_shard(Xt.to(dev), Wgd, W2d, 0, 1, Y, Z, act="swiglu", Wu=Wud)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        Yr, Zr = oracle.mlp_shard(f(Xt), Wg64, W264, 0, 1, "swiglu", Wu=Wu64)
        entry(f"llama70b_decode_tp8_T{T}", f"all {T} token rows", time.perf_counter() - t0,
              [("Y", f(Y), Yr), ("Z", f(Z), Zr)], bf_bar)
    del Wgd, Wud, W2d, Wg64, Wu64, W264

    # simulated TP = 8 block, T = 512: the 8 shards and the reduction on the
    # GPU; the unsharded oracle on 4 rows
    W = synth.WORKLOADS["llama70b_block_sim_tp8"]
    Wg, Wu, W2 = synth.llama_full_weights(W.d, W.k)
    X = synth.llama_tokens(W.T, W.d)
    Yp = torch.empty(W.p, W.T, W.s, dtype=torch.bfloat16, device=dev)
    Zp = torch.empty(W.p, W.T, W.d, device=dev)
    Z = torch.empty(W.T, W.d, device=dev)
    tp.tp_mlp_simulated(X.to(dev), Wg.to(dev), W2.to(dev), W.p, Yp, Zp, Z, act="swiglu",
                        Wu=Wu.to(dev))
    torch.cuda.synchronize()
    rows = [0, 171, 342, W.T - 1]
    Wg64, Wu64, W264 = f(Wg), f(Wu), f(W2)
    t0 = time.perf_counter()
    Zr = oracle.mlp_unsharded(f(X[rows]), Wg64, W264, "swiglu", Wu=Wu64)
    entry(W.name, f"token rows {rows} of {W.T} (unsharded oracle)", time.perf_counter() - t0,
          [("Z", f(Z[rows]), Zr)], bf_bar)
    return out


def cpu_baseline(synth, target_s=12.0):
    """The CPU oracle, untuned, on a bounded sample of the headline workload:
    the first R token rows of one shard forward (rows are independent)."""
    import oracle
    import numpy as np
    import torch

    W = synth.WORKLOADS["llama70b_prefill_tp8"]
    Wg, Wu, W2 = synth.llama_shard_weights(W.d, W.s)
    f = lambda t: t.to(torch.float64).numpy()  # noqa: E731
    Wg, Wu, W2 = f(Wg), f(Wu), f(W2)
    X = f(synth.llama_tokens(W.T, W.d))
    threads = oracle.num_threads()
    # calibrate on one row per thread, then size the sample to ~target_s
    r0 = max(1, threads)
    t0 = time.perf_counter()
    oracle.mlp_shard(X[:r0], Wg, W2, 0, 1, "swiglu", Wu=Wu)
    dt0 = time.perf_counter() - t0
    rows = int(min(W.T, max(r0, r0 * target_s / max(dt0, 1e-6))))
    rows = max(threads, rows - rows % threads)
    t0 = time.perf_counter()
    oracle.mlp_shard(X[:rows], Wg, W2, 0, 1, "swiglu", Wu=Wu)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * W.d * W.s * 3
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu, "wall_s": round(dt, 2),
            "sample": f"first {rows} of {W.T} token rows of one llama70b_prefill_tp8 shard "
                      f"forward (fp64 loops), {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true", help="headline only")
    ap.add_argument("--sections",
                    default="decode,partial_sum,simulated_block,gpt,attention,block,backward,calibration,"
                            "library_gemm",
                    help="comma list of the secondary sections to run (without --quick)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 256 MiB device copy (the reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's shard and runs on one GPU only: the cross-GPU "
              "reduction is out of scope, so there is nothing to time on more.", file=sys.stderr)
        sys.exit(2)

    import torch

    import megatron_tensor_mlp_amd as tp
    from megatron_tensor_mlp_amd import synth

    tp.library()
    log("bench: headline llama70b_prefill_tp8")
    h = headline(torch, tp, synth, args.steps, args.warmup)
    W = h["W"]
    ms = h["total"] / args.steps * 1e3
    value = h["step_flops"] * args.steps / h["total"] / 1e12
    achieved = h["flops_col"] / h["t_col"] / 1e12
    traffic = recorded_traffic("gemm_bf16_tiled_swiglu_llama70b_prefill_tp8")
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": W.name, "T": W.T, "d": W.d, "k": W.k, "p": W.p, "k_per_shard": W.s,
                   "act": W.act, "frac_mfma_peak": round(value / PEAK_BF16_TFLOPS, 4)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel": "gemm_bf16_tiled_kernel<EPI_SWIGLU>",
                     "kernel_us": round(h["t_col"] * 1e6, 2),
                     "flops_per_launch": h["flops_col"]},
        "row_gemm": {"us": round(h["t_row"] * 1e6, 2),
                     "TFLOPs": round(h["flops_row"] / h["t_row"] / 1e12, 2)},
        "timing": {"clock_ramp_s": RAMP_S,
                   "step": dict(h["step_spread"], method="events around each launch of 50 "
                                "steps right after the timed region, eager"),
                   "col_gemm": dict(h["col_spread"], method="the column launch of those steps"),
                   "row_gemm": dict(h["row_spread"], method="the row launch of those steps")},
    }
    sections = set() if args.quick else set(args.sections.split(","))
    if "decode" in sections:
        log("bench: decode")
        result["decode"] = decode_bench(torch, tp, synth, max(5, args.steps // 2), 3)
    if "partial_sum" in sections:
        log("bench: partial sum")
        result["partial_sum"] = partial_sum_bench(torch, tp, max(5, args.steps), 3)
    if "simulated_block" in sections:
        log("bench: simulated block")
        result["simulated_block"] = simulated_block_bench(torch, tp, synth, max(3, args.steps // 4),
                                                          2)
    if "gpt" in sections:
        log("bench: gpt gelu shard")
        result["gpt_gelu_shard"] = gpt_bench(torch, tp, synth, max(5, args.steps // 2), 3)
    if "attention" in sections:
        log("bench: attention projections")
        result["attention_projections"] = attention_bench(torch, tp, synth,
                                                          max(5, args.steps // 2), 3)
    if "block" in sections:
        log("bench: transformer block")
        result["transformer_block"] = transformer_block_bench(torch, tp, synth,
                                                              max(3, args.steps // 10), 2)
    if "backward" in sections:
        log("bench: training step (backward)")
        result["training_step"] = backward_bench(torch, tp, synth, max(5, args.steps // 4), 2)
    if "calibration" in sections:
        log("bench: mfma calibration")
        result["mfma_calibration"] = mfma_calibration(torch, tp)
        log("bench: hbm calibration")
        result["hbm_calibration"] = hbm_calibration(torch, tp, max(5, args.steps // 2), 2)
    if "library_gemm" in sections:
        log("bench: library GEMM reference")
        result["library_gemm_reference"] = library_gemm_reference(torch, synth,
                                                                  max(5, args.steps // 2), 3)
    if "decode" in result:
        d1 = result["decode"]["T1"]
        result["roofline_decode"] = {
            "bound": "hbm", "achieved": d1["GBps"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": d1["frac_hbm"], "traffic": None,
            "kernel": "gemm_bf16_decode_kernel (column step + row step, T = 1)",
            "step_us": d1["us_per_step"], "bytes_per_step": d1["alg_bytes"]}
    if "partial_sum" in result:
        ps = result["partial_sum"]
        result["roofline_partial_sum"] = {
            "bound": "hbm", "achieved": ps["GBps"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": ps["frac_hbm"], "traffic": None, "kernel": "partial_sum_kernel (8 x fp32 "
            "[512, 8192] -> [512, 8192])", "kernel_us": ps["us"], "bytes_per_launch": ps["bytes"]}
    if args.copy_calibration:
        a = torch.empty(64 << 20, device="cuda:0")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(synth)
        if not args.quick:
            log("bench: oracle on every configuration")
            result["cpu_baseline"]["configs"] = oracle_configs(torch, tp, synth)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
