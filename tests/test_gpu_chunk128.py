"""GPU parity of the single-input prefill with 128-token chunks (m3_dims.chunk
= 128) against the fp64 oracle, through the C ABI.  The chunk length only
changes the order in which the GPU sums, never the result, so every case is
held to the same gates as the 64-token chunks: dense calls over ragged
lengths, every single-input shape, both flags, packed sequences (bit for bit
against one dense call per sequence), the B/C preparation, and the SISO
prefill workload's shape."""
import numpy as np
import pytest
import torch

from linear_recurrent_sequence_mamba_amd import binding as m3
from linear_recurrent_sequence_mamba_amd import inputs as I
from oracle import oracle
from tests.util import TOL, cpu64, cuda, rel_err, say

pytestmark = pytest.mark.gpu

KEYS = ("x", "dt", "A", "lam", "theta", "B", "C", "h0", "x_prev", "B_prev")
Q = 128


def _gpu(d, chunk=Q, flags=0, bc=None):
    g = {k: cuda(d[k]) for k in KEYS}
    y, hT = m3.scan_prefill(g["x"], g["dt"], g["A"], g["lam"], g["theta"], g["B"], g["C"],
                            g["h0"], g["x_prev"], g["B_prev"], chunk=chunk, flags=flags, bc=bc)
    torch.cuda.synchronize()
    return y, hT


def _check(w, d, flags=0, heads=None, batches=None):
    y, hT = _gpu(d, flags=flags)
    f = {k: cpu64(d[k]) for k in KEYS}
    yg, hg = cpu64(y), cpu64(hT)
    if heads is not None:
        for k in ("x", "dt", "lam", "theta", "B", "C"):
            f[k] = f[k][batches][:, :, heads]
        f["A"] = f["A"][heads]
        yg, hg = yg[batches][:, :, heads], hg[batches][:, heads]
    ref = oracle.scan(*(f[k] for k in KEYS), flags=flags)
    ey, eh = rel_err(yg, ref.y), rel_err(hg, ref.hT)
    tol = TOL[w.torch_dtype]
    say(f"  y err {ey:.2e}  hT err {eh:.2e}  (tol {tol:.0e})")
    assert ey <= tol and eh <= tol, (ey, eh)


@pytest.mark.parametrize("T", [1, 127, 128, 129, 300])
def test_chunk128_lengths(T):
    w = I.Workload("q", 150, 2, T, 3, 64, 128, 1, Q, "bf16")
    say(f"prefill chunk 128, T={T}")
    _check(w, I.prefill_inputs(w, h0="normal", with_prev=True))


@pytest.mark.parametrize("P,N,dt", [(16, 16, "f32"), (32, 64, "bf16"), (64, 64, "bf16"),
                                    (64, 128, "f32"), (32, 64, "f32")])
def test_chunk128_shapes(P, N, dt):
    w = I.Workload("q", 151, 2, 300, 3, P, N, 1, Q, dt)
    say(f"prefill chunk 128, P={P} N={N} {dt}")
    _check(w, I.prefill_inputs(w, h0="normal", with_prev=True))


@pytest.mark.parametrize("flags", [m3.M3_THETA_IS_ANGLE, m3.M3_A_PER_TOKEN])
def test_chunk128_flags(flags):
    w = I.Workload("q", 152, 2, 260, 3, 64, 128, 1, Q, "bf16")
    d = I.prefill_inputs(w, h0="normal", with_prev=True)
    if flags & m3.M3_A_PER_TOKEN:
        d["A"] = I.token_decay(w, (2, 260))
    say(f"prefill chunk 128, flags={flags}")
    _check(w, d, flags=flags)


def test_chunk128_siso_prefill_workload_sampled():
    """B=4, T=2048, H=32, P=64, N=128 at chunk 128; sampled (batch, head)."""
    w = I.WORKLOADS["siso_prefill"].with_(chunk=Q)
    say("prefill siso_prefill workload, chunk 128")
    _check(w, I.prefill_inputs(w), heads=np.array([0, 17, 31]), batches=np.array([1, 2]))


def test_chunk128_matches_chunk64_and_is_deterministic():
    """Both chunk lengths agree to rounding; equal calls give equal bits."""
    w = I.Workload("q", 153, 2, 400, 3, 64, 128, 1, Q, "bf16")
    d = I.prefill_inputs(w, h0="normal", with_prev=True)
    y1, h1 = _gpu(d, chunk=128)
    y2, h2 = _gpu(d, chunk=128)
    y3, h3 = _gpu(d, chunk=64)
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
    e = max(rel_err(cpu64(y1), cpu64(y3)), rel_err(cpu64(h1), cpu64(h3)))
    say(f"  chunk 128 against chunk 64: {e:.2e}")
    assert e <= 3e-4


def test_chunk128_bcprep_and_deterministic():
    """The B/C preparation at chunk 128 (single rank: the sums of squares of
    a token's B row are combined over eight waves in a fixed order)."""
    w = I.Workload("q", 154, 2, 300, 3, 64, 128, 1, Q, "bf16")
    d, prm = I.bc_prep_inputs(w, I.prefill_inputs(w, h0="normal", with_prev=True))
    bc = m3.BCPrep(**{k: cuda(prm[k]) for k in ("B_weight", "C_weight", "B_bias", "C_bias")},
                   eps=prm["eps"])
    y, hT = _gpu(d, bc=bc)
    y2, h2 = _gpu(d, bc=bc)
    assert torch.equal(y, y2) and torch.equal(hT, h2)
    f = {k: cpu64(d[k]) for k in KEYS}
    H = w.nheads
    for k, which in (("B", "B"), ("C", "C"), ("B_prev", "B")):
        f[k] = oracle.bc_prep(cpu64(d[k]), H, prm[f"{which}_weight"].numpy(),
                              prm[f"{which}_bias"].numpy(), eps=prm["eps"])
    ref = oracle.scan(*(f[k] for k in KEYS))
    ey, eh = rel_err(cpu64(y), ref.y), rel_err(cpu64(hT), ref.hT)
    say(f"  prep, chunk 128: y err {ey:.2e}  hT err {eh:.2e}")
    assert ey <= 3e-3 and eh <= 3e-3


def test_chunk128_packed_sequences():
    """Packed sequences at chunk 128: bit for bit one dense chunk-128 call per
    sequence, and the oracle on each sequence alone."""
    lengths = [0, 1, 127, 128, 129, 260, 0, 7]
    w = I.Workload("q", 155, 1, sum(lengths), 3, 64, 128, 1, Q, "bf16")
    d = I.packed_inputs(w, lengths, h0="normal", with_prev=True)
    g = {k: cuda(v) for k, v in d.items()}
    S, T = len(lengths), sum(lengths)
    y, hT = m3.scan_prefill_varlen(g["cu_seqlens"], g["x"], g["dt"], g["A"], g["lam"], g["theta"],
                                   g["B"], g["C"], g["h0"], g["x_prev"], g["B_prev"], chunk=Q)
    torch.cuda.synchronize()
    cu = [int(v) for v in d["cu_seqlens"]]
    worst = 0.0
    for s in range(S):
        a, b = cu[s], cu[s + 1]
        if a == b:
            assert torch.equal(hT[s], g["h0"][s])
            continue
        e = {k: d[k][a:b].unsqueeze(0).contiguous() for k in ("x", "dt", "lam", "theta", "B", "C")}
        e["A"] = d["A"]
        for k in ("h0", "x_prev", "B_prev"):
            e[k] = d[k][s:s + 1].contiguous()
        yd, hd = _gpu(e)
        assert torch.equal(y[a:b], yd[0]) and torch.equal(hT[s:s + 1], hd), s
        ref = oracle.scan(*(cpu64(e[k]) for k in KEYS))
        worst = max(worst, rel_err(cpu64(yd), ref.y), rel_err(cpu64(hd), ref.hT))
    say(f"  packed, chunk 128: worst err {worst:.2e}")
    assert worst <= 3e-3
