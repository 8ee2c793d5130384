"""Shared helpers for the parity tests: tolerance metric and host copies."""

import numpy as np
import torch

# Tolerances (max-abs error relative to the reference's max-abs, per tensor):
# bf16 inputs with bf16 matrix-core operands and fp32 accumulation: 2e-2;
# fp32 end to end: 1e-4.
TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}


def f64(t):
    """Exact fp64 host copy of a tensor (bf16 and fp32 upcast without rounding)."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()


def rel_err(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = np.abs(ref).max()
    if scale == 0:
        return float(np.abs(x).max())
    return float(np.abs(x - ref).max() / scale)


def rms_rel(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.sqrt(np.mean(ref ** 2))
    return float(np.sqrt(np.mean((x - ref) ** 2)) / den) if den > 0 else 0.0
