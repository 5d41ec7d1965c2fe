"""Shared test helpers: tolerances and conversions (no method arithmetic)."""
import numpy as np
import torch

# Parity bounds for bf16-in / fp32-accumulate paths: relative Frobenius error and
# the largest absolute error relative to the largest reference magnitude.
BF16_REL_FRO = 5e-3
BF16_MAX_REL = 2e-2
# fp32 paths: relative Frobenius error.
F32_REL_FRO = 1e-5


def f64(t):
    """torch tensor (any device/dtype) or array -> fp64 numpy (exact for bf16/fp32)."""
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def errors(got, ref):
    got, ref = f64(got), f64(ref)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite output"
    diff = got - ref
    fro = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300))
    mx = float(np.max(np.abs(diff)) / max(np.max(np.abs(ref)), 1e-300)) if diff.size else 0.0
    return fro, mx


def assert_bf16_close(got, ref, what=""):
    fro, mx = errors(got, ref)
    assert fro <= BF16_REL_FRO and mx <= BF16_MAX_REL, f"{what}: rel_fro={fro:.3e} max_rel={mx:.3e}"
    return fro, mx


def assert_f32_close(got, ref, what=""):
    fro, mx = errors(got, ref)
    assert fro <= F32_REL_FRO, f"{what}: rel_fro={fro:.3e} max_rel={mx:.3e}"
    return fro, mx


def say(*a):
    print(*a, flush=True)
