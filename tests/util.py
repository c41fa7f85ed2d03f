"""Shared test helpers: the error metric and device plumbing."""
from __future__ import annotations

import numpy as np
import torch

# Gates: max relative error (with an RMS floor) for fp32 and bf16 inputs.
TOL = {torch.float32: 1e-5, torch.bfloat16: 3e-3}
# GPU against GPU: two evaluations of one result that round differently (a
# split prefill and the whole one, a decode step after a prefill).  Each is
# within its own rounding of the exact result: fp32 matrix-core operands for
# fp32 inputs; for bf16 inputs bf16 hi + lo operand splits, about 2^-17 per
# operand, chained through two products (measured up to 6e-5 apart).
PAIR_TOL = {torch.float32: 1e-5, torch.bfloat16: 3e-4}


def rel_err(got, ref) -> float:
    """max_i |g_i - o_i| / max(|o_i|, rms(o)) over one output tensor."""
    g = np.asarray(got, dtype=np.float64)
    o = np.asarray(ref, dtype=np.float64)
    assert g.shape == o.shape, (g.shape, o.shape)
    if o.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(o * o)))
    den = np.maximum(np.abs(o), rms if rms > 0 else 1.0)
    return float(np.max(np.abs(g - o) / den))


def cpu64(t):
    if t is None:
        return None
    return t.detach().to("cpu", torch.float64).numpy()


def cuda(t):
    return None if t is None else t.to("cuda").contiguous()


def say(*a):
    print(*a, flush=True)
