"""Seeded synthetic inputs for the Mamba-3 core recurrence.

This module only draws random numbers and shapes them; it holds none of the
recurrence's arithmetic, so both the HIP path and the CPU oracle may use it.

Distributions (one per input, the same for every workload):
  x ~ N(0,1);  dt = softplus(N(0,1));  A = -exp(U(-4,0)) per head;
  lam = sigmoid(N(0,1));  theta ~ U(-pi, pi) per complex pair (or U(0, pi)
  for the one-signed angle-drift stress);  B, C ~ N(0,1), then divided by
  their RMS over the state axis N (per rank column), which stands in for the
  RMS normalisation of B and C that the pages place in front of the core
  [xxxxx.co.kr Mamba-3 article, section 2 (BC/QK normalisation)].
The activations are applied here because the library takes dt and lam
already activated.

Every array is drawn in float32 from numpy's PCG64 ``default_rng([cfg_id,
stream])`` and then cast to the workload's input dtype with torch (bf16 or
fp32); the rounded tensors are THE inputs for both sides.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    rank: int = 1
    chunk: int = 64
    dtype: str = "bf16"          # input dtype of x, B, C, dt, lam, theta
    h0: str = "zero"             # "zero" or "normal"
    steps: int = 0               # decode workloads: number of sequential steps
    theta_dist: str = "pm_pi"    # "pm_pi" = U(-pi,pi), "pos_pi" = U(0,pi)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads: tiny parity shape, SISO chunked prefill, SISO decode,
# MIMO rank-4 decode, MIMO rank-4 long prefill.
WORKLOADS = {
    "tiny": Workload("tiny", 0, 1, 64, 2, 16, 16, 1, 64, "f32", "zero"),
    "siso_prefill": Workload("siso_prefill", 1, 4, 2048, 32, 64, 128, 1, 64, "bf16", "zero"),
    "siso_decode": Workload("siso_decode", 2, 128, 1, 64, 64, 128, 1, 64, "bf16", "normal", 1000),
    "mimo_decode": Workload("mimo_decode", 3, 128, 1, 64, 64, 128, 4, 64, "bf16", "normal", 1000),
    "mimo_prefill": Workload("mimo_prefill", 4, 1, 16384, 64, 64, 128, 4, 64, "bf16", "zero"),
}


# Packed serving mixes: the two prefill shapes with their tokens split into
# sequences whose lengths are drawn uniformly from 1..4096 (the article's
# Table 7 times prompts of 512 to 16384 tokens; this draw averages about
# 2048 and leaves almost every sequence with a ragged last chunk).
PACKED = {
    "siso_prefill_varlen": (Workload("siso_prefill_varlen", 5, 1, 8192, 32, 64, 128, 1, 64, "bf16",
                                     "zero"), 4096),
    "mimo_prefill_varlen": (Workload("mimo_prefill_varlen", 6, 1, 16384, 64, 64, 128, 4, 64, "bf16",
                                     "zero"), 4096),
}


def packed_lengths(w: Workload, max_len: int) -> list:
    """Sequence lengths U{1..max_len} from ``default_rng([cfg_id, 0x1E5])``
    until they fill w.seqlen tokens (the last one is cut to fit)."""
    rng = np.random.default_rng([w.cfg_id, 0x1E5])
    out, left = [], w.seqlen
    while left > 0:
        n = min(int(rng.integers(1, max_len + 1)), left)
        out.append(n)
        left -= n
    return out


def packed_inputs(w: Workload, lengths, stream: int = 0, h0: str | None = None,
                  with_prev: bool = False) -> dict:
    """Inputs of a packed-sequence prefill: the token arrays of ``w`` (batch
    1, seqlen = sum(lengths)) without their batch axis, the offsets
    ``cu_seqlens`` (int32, len(lengths) + 1), and one h0 / x_prev / B_prev row
    per sequence.  Lengths may be 0."""
    assert w.batch == 1 and sum(lengths) == w.seqlen
    tok = prefill_inputs(w, stream=stream)
    out = {k: v[0] for k, v in tok.items() if k not in ("A", "h0", "x_prev", "B_prev")}
    out["A"] = tok["A"]
    per = prefill_inputs(w.with_(batch=len(lengths), seqlen=1), stream=stream + 500, h0=h0,
                         with_prev=with_prev)
    for k in ("h0", "x_prev", "B_prev"):
        out[k] = per[k]
    out["cu_seqlens"] = torch.from_numpy(
        np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32))
    return out


def bc_prep_inputs(w: Workload, d: dict, stream: int = 0, eps: float = 1e-6):
    """Inputs of the in-kernel B/C preparation for the tensors of ``d``
    (prefill or token layouts, B/C with their group axis third from the end):
    B and C (and B_prev) become raw projections by a scale U(0.2, 5) per
    token, group and rank column, cast back to the input dtype; the weights
    are U(0.5, 1.5) [N] and the per-head biases N(0, 0.5^2) [H, N, R], fp32.
    Returns (d2, params) with params = dict(B_weight, C_weight, B_bias, C_bias,
    eps) as CPU tensors."""
    rng = np.random.default_rng([w.cfg_id, 0xBC, stream])
    f32 = np.float32
    out = dict(d)
    for k in ("B", "C", "B_prev"):
        v = d.get(k)
        if v is None:
            continue
        shape = tuple(v.shape[:-2]) + (1, v.shape[-1])
        sc = rng.uniform(0.2, 5.0, size=shape).astype(f32)
        out[k] = _cast(v.to(torch.float32).numpy() * sc, v.dtype)
    N, H, R = w.dstate, w.nheads, w.rank
    params = dict(
        B_weight=torch.from_numpy(rng.uniform(0.5, 1.5, size=N).astype(f32)),
        C_weight=torch.from_numpy(rng.uniform(0.5, 1.5, size=N).astype(f32)),
        B_bias=torch.from_numpy((rng.standard_normal((H, N, R)) * 0.5).astype(f32)),
        C_bias=torch.from_numpy((rng.standard_normal((H, N, R)) * 0.5).astype(f32)),
        eps=eps)
    return out, params


def _softplus(v):
    return np.logaddexp(np.float32(0.0), v).astype(np.float32)


def _sigmoid(v):
    return (1.0 / (1.0 + np.exp(-v))).astype(np.float32)


def _rms_normalise(v, axis):
    rms = np.sqrt(np.mean(np.square(v, dtype=np.float32), axis=axis, keepdims=True))
    return (v / np.maximum(rms, np.float32(1e-12))).astype(np.float32)


def _cast(a: np.ndarray, dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype).contiguous()


def _draw_common(rng, lead, H, P, N, R, theta_dist):
    """Draw x, dt, lam, theta, B, C for leading shape ``lead`` (+ H)."""
    f32 = np.float32
    x = rng.standard_normal(lead + (H, P, R), dtype=f32)
    dt = _softplus(rng.standard_normal(lead + (H,), dtype=f32))
    lam = _sigmoid(rng.standard_normal(lead + (H,), dtype=f32))
    if theta_dist == "pos_pi":
        theta = (rng.random(lead + (H, N // 2), dtype=f32) * f32(math.pi)).astype(f32)
    else:
        theta = ((rng.random(lead + (H, N // 2), dtype=f32) * 2 - 1) * f32(math.pi)).astype(f32)
    B = _rms_normalise(rng.standard_normal(lead + (H, N, R), dtype=f32), axis=-2)
    C = _rms_normalise(rng.standard_normal(lead + (H, N, R), dtype=f32), axis=-2)
    return x, dt, lam, theta, B, C


def head_decay(w: Workload) -> torch.Tensor:
    """A = -exp(U(-4, 0)), one per head, fp32."""
    rng = np.random.default_rng([w.cfg_id, 0x0A])
    return torch.from_numpy(-np.exp(rng.uniform(-4.0, 0.0, size=(w.nheads,))).astype(np.float32))


def token_decay(w: Workload, lead: tuple, stream: int = 0) -> torch.Tensor:
    """A drawn independently for every leading index (tokens, or (batch,
    head) pairs of a decode step): -exp(U(-4, 0)), fp32, shape lead + (H,)."""
    rng = np.random.default_rng([w.cfg_id, 0x0A7, stream])
    return torch.from_numpy(-np.exp(rng.uniform(-4.0, 0.0, size=tuple(lead) + (w.nheads,)))
                            .astype(np.float32))


def theta_proj_inputs(w: Workload, lead: tuple, dim: int, groups: int | None = None,
                      stream: int = 0):
    """Inputs of the in-kernel angle projection: u ~ N(0, 1) of shape lead +
    (dim,) and W ~ N(0, (pi / 2)^2 / dim) of shape [G, N/2, dim] (so the
    angles come out ~N(0, (pi/2)^2), the spread of U(-pi, pi)), cast to the
    input dtype.  Returns (u, W) as CPU tensors."""
    rng = np.random.default_rng([w.cfg_id, 0x7E, stream])
    G = groups or w.nheads
    u = rng.standard_normal(tuple(lead) + (dim,), dtype=np.float32)
    W = (rng.standard_normal((G, w.dstate // 2, dim), dtype=np.float32)
         * np.float32(0.5 * math.pi / math.sqrt(dim)))
    return _cast(u, w.torch_dtype), _cast(W, w.torch_dtype)


def prefill_inputs(w: Workload, stream: int = 0, h0: str | None = None,
                   with_prev: bool = False) -> dict:
    """Inputs of one prefill call as CPU torch tensors (input dtype; A, h0 fp32).

    ``h0`` overrides the workload's initial-state kind ("zero"/"normal");
    ``with_prev`` also draws the token before the first one (x_prev, B_prev).
    """
    rng = np.random.default_rng([w.cfg_id, 1000 + stream])
    Bsz, T, H, P, N, R = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.rank
    x, dt, lam, theta, B, C = _draw_common(rng, (Bsz, T), H, P, N, R, w.theta_dist)
    td = w.torch_dtype
    out = dict(x=_cast(x, td), dt=_cast(dt, td), lam=_cast(lam, td),
               theta=_cast(theta, td), B=_cast(B, td), C=_cast(C, td),
               A=head_decay(w))
    kind = h0 or w.h0
    if kind == "normal":
        out["h0"] = torch.from_numpy(rng.standard_normal((Bsz, H, P, N), dtype=np.float32))
    else:
        out["h0"] = None
    if with_prev:
        xp, _, _, _, Bp, _ = _draw_common(rng, (Bsz,), H, P, N, R, w.theta_dist)
        out["x_prev"] = _cast(xp, td)
        out["B_prev"] = _cast(Bp, td)
    else:
        out["x_prev"] = None
        out["B_prev"] = None
    return out


def decode_state(w: Workload) -> torch.Tensor:
    """Initial decode state h ~ N(0,1), fp32 [Bsz,H,P,N]."""
    rng = np.random.default_rng([w.cfg_id, 0x5EED])
    return torch.from_numpy(rng.standard_normal(
        (w.batch, w.nheads, w.headdim, w.dstate), dtype=np.float32))


def decode_step_inputs(w: Workload, step: int) -> dict:
    """Fresh inputs of decode step ``step`` (x_t, B_t, C_t, dt_t, lam_t,
    theta_t in the input dtype), from ``default_rng([cfg_id, 1 + step])``.
    The previous token's x and B are those of step - 1 (zero before step 0
    unless the caller supplies them)."""
    rng = np.random.default_rng([w.cfg_id, 1 + step])
    x, dt, lam, theta, B, C = _draw_common(rng, (w.batch,), w.nheads, w.headdim,
                                           w.dstate, w.rank, w.theta_dist)
    td = w.torch_dtype
    return dict(x=_cast(x, td), dt=_cast(dt, td), lam=_cast(lam, td),
                theta=_cast(theta, td), B=_cast(B, td), C=_cast(C, td))


def to_f64(t):
    """Exact upcast of a (rounded) input tensor to a float64 numpy array."""
    if t is None:
        return None
    return t.detach().to("cpu", torch.float64).numpy()
