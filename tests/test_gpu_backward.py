"""GPU parity of m3_scan_prefill_backward (the gradients of the prefill scan)
against the fp64 oracle's adjoint (oracle.scan_backward, itself pinned by
finite differences of the forward scan).

Gates.  bf16 inputs: the forward's 3e-3 for every gradient.  fp32 inputs: the
forward's 1e-5 for the gradients that are elementwise products of chunk
contractions (x, B, C, lam, h0, x_prev, B_prev), and 2e-5 for dt, A and
theta: each of those is a suffix sum over the chunk's tokens (up to 64
terms, then carried from chunk to chunk) of terms that carry the
elementwise gradients' own rounding, so its error can reach about twice
theirs (measured up to 8.7e-6, against up to 6.4e-6 for the others).  Both
sides take the same rounded inputs; the measured errors are printed."""
import numpy as np
import pytest
import torch

from linear_recurrent_sequence_mamba_amd import binding as m3
from linear_recurrent_sequence_mamba_amd import inputs as I
from oracle import oracle
from tests.util import PAIR_TOL, cpu64, cuda, rel_err, say

pytestmark = pytest.mark.gpu

GTOL = {torch.float32: 1e-5, torch.bfloat16: 3e-3}
# fp32 inputs: the suffix-summed gradients (see the module docstring)
GTOL_SUFFIX32 = {"dt": 2e-5, "A": 2e-5, "theta": 2e-5}
KEYS = ("x", "dt", "A", "lam", "theta", "B", "C", "h0", "x_prev", "B_prev")


def _cotangents(w, d, seed=0, dhT=True):
    rng = np.random.default_rng([w.cfg_id, 0xD7, seed])
    dy = torch.from_numpy(rng.standard_normal(tuple(d["x"].shape), dtype=np.float32))
    dh = torch.from_numpy(rng.standard_normal((w.batch, w.nheads, w.headdim, w.dstate),
                                              dtype=np.float32)) if dhT else None
    return dy, dh


def _per_head(t, H, dim):
    return t if t is None or t.shape[dim] == H else t.repeat_interleave(H // t.shape[dim], dim=dim)


def _group_sum(g, G, dim):
    """Sum a per-head gradient over the heads of each group."""
    if g is None or g.shape[dim] == G:
        return g
    s = list(g.shape)
    s[dim:dim + 1] = [G, s[dim] // G]
    return g.reshape(s).sum(axis=dim + 1)


def _oracle(d, dy, dhT, flags=0):
    H = d["x"].shape[2]
    G = d["B"].shape[2]
    e = {k: cpu64(d[k]) for k in KEYS}
    for k in ("B", "C", "theta"):
        e[k] = cpu64(_per_head(d[k], H, 2))
    e["B_prev"] = cpu64(_per_head(d["B_prev"], H, 1))
    g = oracle.scan_backward(*(e[k] for k in KEYS), dy=cpu64(dy), dhT=cpu64(dhT), flags=flags)
    for k in ("B", "C", "theta"):
        g[k] = _group_sum(g[k], G, 2)
    g["B_prev"] = _group_sum(g["B_prev"], G, 1)
    return g


def _gpu(d, dy, dhT, flags=0):
    g = {k: cuda(v) for k, v in d.items()}
    out = m3.scan_prefill_backward(g["x"], g["dt"], g["A"], g["lam"], g["theta"], g["B"], g["C"],
                                   cuda(dy), h0=g["h0"], x_prev=g["x_prev"], B_prev=g["B_prev"],
                                   dhT=cuda(dhT), flags=flags)
    torch.cuda.synchronize()
    return out


def _check(w, d, dy, dhT, flags=0, tol=None):
    got = _gpu(d, dy, dhT, flags)
    ref = _oracle(d, dy, dhT, flags)
    tol = tol or GTOL[w.torch_dtype]
    errs = {}
    for k in KEYS:
        if ref[k] is None:
            assert got.get(k) is None
            continue
        errs[k] = rel_err(cpu64(got[k]), ref[k])
    say("  " + "  ".join(f"d{k} {v:.1e}" for k, v in errs.items()) + f"  (tol {tol:.0e})")
    gate = lambda k: max(tol, GTOL_SUFFIX32.get(k, 0.0)) if w.torch_dtype == torch.float32 else tol
    bad = {k: v for k, v in errs.items() if not v <= gate(k)}
    assert not bad, bad


@pytest.mark.parametrize("T", [1, 63, 64, 65, 130])
def test_backward_lengths(T):
    w = I.Workload("g", 130, 2, T, 3, 64, 128, 1, 64, "bf16")
    d = I.prefill_inputs(w, h0="normal", with_prev=True)
    dy, dhT = _cotangents(w, d)
    say(f"backward T={T}")
    _check(w, d, dy, dhT)


@pytest.mark.parametrize("P,N,dt", [(16, 16, "f32"), (32, 64, "bf16"), (64, 64, "bf16"),
                                    (64, 128, "f32"), (32, 64, "f32")])
def test_backward_shapes(P, N, dt):
    w = I.Workload("g", 131, 2, 150, 2, P, N, 1, 64, dt)
    d = I.prefill_inputs(w, h0="normal", with_prev=True)
    dy, dhT = _cotangents(w, d)
    say(f"backward P={P} N={N} {dt}")
    _check(w, d, dy, dhT)


def test_backward_variants():
    w = I.Workload("g", 132, 2, 140, 4, 64, 128, 1, 64, "bf16")
    base = I.prefill_inputs(w, h0="normal", with_prev=True)
    dy, dhT = _cotangents(w, base)
    say("backward, head groups G=2")
    d = dict(base)
    for k in ("B", "C", "theta"):
        d[k] = base[k][:, :, :2].contiguous()
    d["B_prev"] = base["B_prev"][:, :2].contiguous()
    _check(w, d, dy, dhT)
    say("backward, no h0, no previous token, no dhT")
    d = I.prefill_inputs(w, h0="zero", with_prev=False)
    _check(w, d, dy, None)
    say("backward, theta is the angle")
    _check(w, base, dy, dhT, flags=m3.M3_THETA_IS_ANGLE)
    say("backward, A per token")
    d = dict(base)
    rng = np.random.default_rng(5)
    d["A"] = torch.from_numpy(-np.exp(rng.uniform(-4, 0, size=(2, 140, 4))).astype(np.float32))
    _check(w, d, dy, dhT, flags=m3.M3_A_PER_TOKEN)
    say("backward, bf16 dy")
    _check(w, base, dy.to(torch.bfloat16), dhT)


@pytest.mark.parametrize("P,N,R,dt", [(64, 128, 2, "bf16"), (64, 128, 4, "f32"), (32, 64, 4, "bf16"),
                                      (64, 64, 4, "f32")])
def test_backward_mimo_shapes(P, N, R, dt):
    """Rank R > 1: every token is R columns of x, B and C; the gradients of
    every rank against the oracle's (which runs the rank-R recurrence)."""
    w = I.Workload("g", 134, 2, 150, 2, P, N, R, 64, dt)
    d = I.prefill_inputs(w, h0="normal", with_prev=True)
    dy, dhT = _cotangents(w, d)
    say(f"backward P={P} N={N} R={R} {dt}")
    _check(w, d, dy, dhT)


@pytest.mark.parametrize("T", [1, 64, 97])
def test_backward_mimo_lengths(T):
    w = I.Workload("g", 135, 1, T, 2, 64, 128, 4, 64, "bf16")
    d = I.prefill_inputs(w, h0="normal", with_prev=True)
    dy, dhT = _cotangents(w, d)
    say(f"backward R=4 T={T}")
    _check(w, d, dy, dhT)


def test_backward_mimo_variants():
    w = I.Workload("g", 136, 2, 140, 4, 64, 128, 4, 64, "bf16")
    base = I.prefill_inputs(w, h0="normal", with_prev=True)
    dy, dhT = _cotangents(w, base)
    say("backward R=4, head groups G=2")
    d = dict(base)
    for k in ("B", "C", "theta"):
        d[k] = base[k][:, :, :2].contiguous()
    d["B_prev"] = base["B_prev"][:, :2].contiguous()
    _check(w, d, dy, dhT)
    say("backward R=4, no h0, no previous token, no dhT")
    d = I.prefill_inputs(w, h0="zero", with_prev=False)
    _check(w, d, dy, None)
    say("backward R=4, theta is the angle, A per token, bf16 dy")
    d = dict(base)
    rng = np.random.default_rng(6)
    d["A"] = torch.from_numpy(-np.exp(rng.uniform(-4, 0, size=(2, 140, 4))).astype(np.float32))
    _check(w, d, dy.to(torch.bfloat16), dhT, flags=m3.M3_THETA_IS_ANGLE | m3.M3_A_PER_TOKEN)


@pytest.mark.parametrize("R", [1, 4])
def test_backward_bf16_operand_range(R):
    """bf16 inputs with x scaled by 1e4 and B, C by 1e-3: the bf16 hi + lo
    matrix-core operands keep fp32's range, so the gate is unchanged."""
    w = I.Workload("g", 137, 2, 150, 2, 64, 128, R, 64, "bf16")
    d = I.prefill_inputs(w, h0="normal", with_prev=True)
    scale = lambda t, c: (t.to(torch.float32) * c).to(torch.bfloat16)
    for k, c in (("x", 1e4), ("x_prev", 1e4), ("B", 1e-3), ("B_prev", 1e-3), ("C", 1e-3)):
        d[k] = scale(d[k], c)
    dy, dhT = _cotangents(w, d)
    say(f"backward bf16 range R={R}")
    _check(w, d, dy, dhT)


@pytest.mark.parametrize("R", [1, 4])
def test_backward_is_deterministic_and_matches_split(R):
    """Two calls give identical gradients; the h0 gradient of the second half
    of a split scan is the dhT that the first half's backward needs."""
    w = I.Workload("g", 133, 2, 200, 3, 64, 128, R, 64, "bf16")
    d = I.prefill_inputs(w, h0="normal", with_prev=True)
    dy, dhT = _cotangents(w, d)
    g1 = _gpu(d, dy, dhT)
    g2 = _gpu(d, dy, dhT)
    assert all(torch.equal(g1[k], g2[k]) for k in g1 if g1[k] is not None)
    k = 90
    cut = lambda t, a, b: t[:, a:b].contiguous()
    d2 = {kk: (cut(v, k, 200) if kk in ("x", "dt", "lam", "theta", "B", "C") else v) for kk, v in d.items()}
    gd = {kk: cuda(v) for kk, v in d.items()}
    d1 = {kk: (cut(v, 0, k) if kk in ("x", "dt", "lam", "theta", "B", "C") else v) for kk, v in d.items()}
    # the first half's final state and last token feed the second half
    _, h1 = m3.scan_prefill(*(cuda(d1[kk]) for kk in ("x", "dt", "A", "lam", "theta", "B", "C")),
                            gd["h0"], gd["x_prev"], gd["B_prev"])
    d2.update(h0=h1.cpu(), x_prev=d["x"][:, k - 1].contiguous(), B_prev=d["B"][:, k - 1].contiguous())
    gb = _gpu(d2, cut(dy, k, 200), dhT)
    ga = _gpu(d1, cut(dy, 0, k), gb["h0"].cpu())
    # x and B of token k - 1 also feed the second half as its token before
    gx = torch.cat([ga["x"], gb["x"]], 1)
    gx[:, k - 1] += gb["x_prev"]
    gB = torch.cat([ga["B"], gb["B"]], 1)
    gB[:, k - 1] += gb["B_prev"]
    e = rel_err(cpu64(gx), cpu64(g1["x"]))
    eb = rel_err(cpu64(gB), cpu64(g1["B"]))
    say(f"  split: dx err {e:.1e}  dB err {eb:.1e}")
    # GPU against GPU: both round differently (bf16 operand splits)
    assert e <= PAIR_TOL[w.torch_dtype] and eb <= PAIR_TOL[w.torch_dtype]


@pytest.mark.parametrize("name", ["siso_prefill", "mimo_prefill"])
def test_backward_full_workload_sampled(name):
    """The prefill workloads (SISO B=4, T=2048, H=32; MIMO B=1, T=16384,
    H=64, R=4) in the launch configuration of the benchmark; the gradients of
    sampled (batch, head) pairs against the oracle."""
    w = I.WORKLOADS[name]
    d = I.prefill_inputs(w)
    dy, dhT = _cotangents(w, d, dhT=False)
    say(f"backward {name}")
    got = _gpu(d, dy, None)
    for b, h in ((0, 0), (w.batch - 1, 17)):
        sub = {k: (v[b:b + 1, :, h:h + 1].contiguous() if k in ("x", "dt", "lam", "theta", "B", "C")
                   else v) for k, v in d.items()}
        sub["A"] = d["A"][h:h + 1]
        ref = _oracle(sub, dy[b:b + 1, :, h:h + 1].contiguous(), None)
        for k in ("x", "dt", "lam", "theta", "B", "C"):
            e = rel_err(cpu64(got[k][b:b + 1, :, h:h + 1]), ref[k])
            say(f"  ({b},{h}) d{k} {e:.1e}")
            assert e <= GTOL[torch.bfloat16], (k, e)
