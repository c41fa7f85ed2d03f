"""GPU parity of the in-kernel angle projection (m3_dims.tp: theta = W u per
token row and head group, made inside the prefill chunk kernels and the
decode step) against the fp64 oracle: oracle.theta_proj makes the angles from
the same u and W, then the oracle's scan or decode step runs on them."""
import numpy as np
import pytest
import torch

from linear_recurrent_sequence_mamba_amd import binding as m3
from linear_recurrent_sequence_mamba_amd import inputs as I
from oracle import oracle
from tests.util import TOL, cpu64, cuda, rel_err, say

pytestmark = pytest.mark.gpu

KEYS = ("x", "dt", "A", "lam", "theta", "B", "C", "h0", "x_prev", "B_prev")


def _per_head(t, H, dim):
    return t if t is None or t.shape[dim] == H else t.repeat_interleave(H // t.shape[dim], dim=dim)


def _prefill_case(w, D, groups=None, seed=0):
    d = I.prefill_inputs(w, stream=seed, h0="normal", with_prev=True)
    G = groups or w.nheads
    if groups is not None:
        for k in ("B", "C"):
            d[k] = d[k][:, :, :G].contiguous()
        d["B_prev"] = d["B_prev"][:, :G].contiguous()
    u, W = I.theta_proj_inputs(w, (w.batch, w.seqlen), D, G, stream=seed)
    return d, u, W


def _oracle_prefill(d, u, W, flags=0, bc=None):
    H = d["x"].shape[2]
    f = {k: cpu64(d[k]) for k in KEYS}
    f["theta"] = oracle.theta_proj(cpu64(u), cpu64(W))           # [Bsz, T, G, N/2]
    f["theta"] = np.repeat(f["theta"], H // f["theta"].shape[2], axis=2)
    for k, ax in (("B", 2), ("C", 2), ("B_prev", 1)):
        if bc is None:
            f[k] = cpu64(_per_head(d[k], H, ax))
        else:
            which = "C" if k == "C" else "B"
            f[k] = oracle.bc_prep(cpu64(d[k]), H, bc[f"{which}_weight"].numpy(),
                                  bc[f"{which}_bias"].numpy(), eps=bc["eps"])
    return oracle.scan(*(f[k] for k in KEYS), flags=flags)


def _gpu_prefill(d, u, W, chunk=0, flags=0, bc=None):
    g = {k: cuda(d[k]) for k in KEYS}
    tp = m3.ThetaProj(cuda(u), cuda(W))
    bcp = None
    if bc is not None:
        bcp = m3.BCPrep(**{k: cuda(bc[k]) for k in ("B_weight", "C_weight", "B_bias", "C_bias")},
                        eps=bc["eps"])
    y, hT = m3.scan_prefill(g["x"], g["dt"], g["A"], g["lam"], None, g["B"], g["C"], g["h0"],
                            g["x_prev"], g["B_prev"], chunk=chunk, flags=flags, tp=tp, bc=bcp)
    torch.cuda.synchronize()
    return y, hT


def _check(w, y, hT, ref):
    ey, eh = rel_err(cpu64(y), ref.y), rel_err(cpu64(hT), ref.hT)
    tol = TOL[w.torch_dtype]
    say(f"  y err {ey:.2e}  hT err {eh:.2e}  (tol {tol:.0e})")
    assert ey <= tol and eh <= tol, (ey, eh)


@pytest.mark.parametrize("P,N,R,dt,D", [
    (64, 128, 1, "bf16", 64), (64, 128, 4, "bf16", 96), (16, 16, 1, "f32", 32),
    (64, 128, 1, "f32", 64), (64, 64, 4, "bf16", 32), (64, 128, 2, "bf16", 160),
])
def test_prefill_projection(P, N, R, dt, D):
    w = I.Workload("tp", 160, 2, 150, 3, P, N, R, 64, dt)
    d, u, W = _prefill_case(w, D)
    say(f"prefill projection P={P} N={N} R={R} {dt} D={D}")
    _check(w, *_gpu_prefill(d, u, W), _oracle_prefill(d, u, W))


def test_prefill_projection_variants():
    w = I.Workload("tp", 161, 2, 200, 4, 64, 128, 1, 64, "bf16")
    d, u, W = _prefill_case(w, 64, groups=2)
    say("prefill projection, head groups G=2")
    _check(w, *_gpu_prefill(d, u, W), _oracle_prefill(d, u, W))
    say("prefill projection, theta as the angle")
    _check(w, *_gpu_prefill(d, u, W, flags=m3.M3_THETA_IS_ANGLE),
           _oracle_prefill(d, u, W, flags=m3.M3_THETA_IS_ANGLE))
    say("prefill projection, chunk 128")
    _check(w, *_gpu_prefill(d, u, W, chunk=128), _oracle_prefill(d, u, W))
    say("prefill projection with the B/C preparation")
    dp, prm = I.bc_prep_inputs(w, d)
    _check(w, *_gpu_prefill(dp, u, W, bc=prm), _oracle_prefill(dp, u, W, bc=prm))


def test_prefill_projection_long_mimo_sampled():
    """The MIMO rank-4 long prefill shape (T = 16384) with the projection,
    sampled heads against the oracle."""
    w = I.WORKLOADS["mimo_prefill"].with_(nheads=16)
    d, u, W = _prefill_case(w, 64)
    y, hT = _gpu_prefill(d, u, W)
    heads = np.array([0, 11])
    e = {k: d[k] for k in KEYS}
    for k in ("x", "dt", "lam", "B", "C"):
        e[k] = d[k][:, :, heads]
    e["A"] = d["A"][heads]
    e["h0"] = d["h0"][:, heads]
    e["x_prev"], e["B_prev"] = d["x_prev"][:, heads], d["B_prev"][:, heads]
    ref = _oracle_prefill(e, u, W[heads])
    say("prefill projection, long MIMO shape")
    _check(w, y[:, :, heads], hT[:, heads], ref)


def test_varlen_projection():
    lengths = [0, 1, 63, 64, 65, 200, 7]
    w = I.Workload("tp", 162, 1, sum(lengths), 3, 64, 128, 4, 64, "bf16")
    pk = I.packed_inputs(w, lengths, h0="normal", with_prev=True)
    u, W = I.theta_proj_inputs(w, (sum(lengths),), 64)
    g = {k: cuda(v) for k, v in pk.items()}
    y, hT = m3.scan_prefill_varlen(g["cu_seqlens"], g["x"], g["dt"], g["A"], g["lam"], None,
                                   g["B"], g["C"], g["h0"], g["x_prev"], g["B_prev"],
                                   tp=m3.ThetaProj(cuda(u), cuda(W)))
    torch.cuda.synchronize()
    cu = [int(v) for v in pk["cu_seqlens"]]
    worst = 0.0
    for s in range(len(lengths)):
        a, b = cu[s], cu[s + 1]
        if a == b:
            continue
        e = {k: pk[k][a:b].unsqueeze(0) for k in ("x", "dt", "lam", "B", "C")}
        e.update(A=pk["A"], theta=None, h0=pk["h0"][s:s + 1], x_prev=pk["x_prev"][s:s + 1],
                 B_prev=pk["B_prev"][s:s + 1])
        ref = _oracle_prefill(e, u[a:b].unsqueeze(0), W)
        worst = max(worst, rel_err(cpu64(y[a:b]), ref.y[0]), rel_err(cpu64(hT[s:s + 1]), ref.hT))
    say(f"  packed with projection: worst err {worst:.2e}")
    assert worst <= 3e-3


@pytest.mark.parametrize("P,N,R,dt,D", [
    (64, 128, 1, "bf16", 64), (64, 128, 4, "bf16", 96), (16, 16, 1, "f32", 32),
    (64, 128, 4, "f32", 64), (48, 256, 1, "bf16", 32), (32, 64, 2, "bf16", 128),
])
def test_decode_projection(P, N, R, dt, D):
    """Three decode steps, each with the projection, against the oracle."""
    w = I.Workload("tp", 163, 3, 1, 4, P, N, R, 64, dt, "normal")
    h_cpu = I.decode_state(w)
    h = cuda(h_cpu)
    href = cpu64(h_cpu)
    A = I.head_decay(w)
    say(f"decode projection P={P} N={N} R={R} {dt} D={D}")
    prev = None
    ey = 0.0
    for s in range(3):
        d = I.decode_step_inputs(w, s)
        u, W = I.theta_proj_inputs(w, (w.batch,), D, stream=s)
        g = {k: cuda(v) for k, v in d.items()}
        y = m3.decode_step(h, g["x"], g["B"], g["C"], g["dt"], cuda(A), g["lam"], None,
                           x_prev=None if prev is None else cuda(prev["x"]),
                           B_prev=None if prev is None else cuda(prev["B"]),
                           tp=m3.ThetaProj(cuda(u), cuda(W)))
        th = oracle.theta_proj(cpu64(u), cpu64(W))                # [Bsz, G, N/2]
        yr, href = oracle.decode_step(href, cpu64(d["x"]), None if prev is None else cpu64(prev["x"]),
                                      cpu64(d["B"]), None if prev is None else cpu64(prev["B"]),
                                      cpu64(d["C"]), cpu64(d["dt"]), cpu64(A), cpu64(d["lam"]), th)
        torch.cuda.synchronize()
        ey = max(ey, rel_err(cpu64(y), yr))
        prev = d
    eh = rel_err(cpu64(h), href)
    tol = TOL[w.torch_dtype]
    say(f"  y err {ey:.2e}  h err {eh:.2e}  (tol {tol:.0e})")
    assert ey <= tol and eh <= tol, (ey, eh)


def test_decode_projection_groups_and_prep():
    """Head groups (G = 2 of 4) with the projection and the B/C preparation."""
    w = I.Workload("tp", 164, 2, 1, 4, 64, 128, 4, 64, "bf16", "normal")
    G = 2
    h_cpu = I.decode_state(w)
    h = cuda(h_cpu)
    A = I.head_decay(w)
    d = I.decode_step_inputs(w, 0)
    for k in ("B", "C"):
        d[k] = d[k][:, :G].contiguous()
    dp, prm = I.bc_prep_inputs(w, {k: d[k] for k in ("B", "C")})
    u, W = I.theta_proj_inputs(w, (w.batch,), 64, G)
    bc = m3.BCPrep(**{k: cuda(prm[k]) for k in ("B_weight", "C_weight", "B_bias", "C_bias")},
                   eps=prm["eps"])
    y = m3.decode_step(h, cuda(d["x"]), cuda(dp["B"]), cuda(dp["C"]), cuda(d["dt"]), cuda(A),
                       cuda(d["lam"]), None, bc=bc, tp=m3.ThetaProj(cuda(u), cuda(W)))
    th = np.repeat(oracle.theta_proj(cpu64(u), cpu64(W)), 2, axis=1)
    Bh = oracle.bc_prep(cpu64(dp["B"]), 4, prm["B_weight"].numpy(), prm["B_bias"].numpy(),
                        eps=prm["eps"])
    Ch = oracle.bc_prep(cpu64(dp["C"]), 4, prm["C_weight"].numpy(), prm["C_bias"].numpy(),
                        eps=prm["eps"])
    yr, hr = oracle.decode_step(cpu64(h_cpu), cpu64(d["x"]), None, Bh, None, Ch, cpu64(d["dt"]),
                                cpu64(A), cpu64(d["lam"]), th)
    torch.cuda.synchronize()
    ey, eh = rel_err(cpu64(y), yr), rel_err(cpu64(h), hr)
    say(f"decode projection, groups and prep: y err {ey:.2e}  h err {eh:.2e}")
    assert ey <= 3e-3 and eh <= 3e-3
