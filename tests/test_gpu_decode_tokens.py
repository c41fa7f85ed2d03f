"""GPU parity of m3_decode_tokens (K decode steps in one call) against the fp64
oracle's scan over the same K tokens from the same state, and against K calls
of m3_decode_step."""
import numpy as np
import pytest
import torch

from linear_recurrent_sequence_mamba_amd import binding as m3
from linear_recurrent_sequence_mamba_amd import inputs as I
from oracle import oracle
from tests.util import TOL, cpu64, cuda, rel_err, say

pytestmark = pytest.mark.gpu


def _inputs(w, prev=True, groups=None):
    """K tokens (w.seqlen) drawn like a prefill, a random entry state, and the
    token before the first; with `groups`, B, C and theta keep that many head
    slots."""
    d = I.prefill_inputs(w, h0="normal", with_prev=prev)
    if groups is not None:
        for k in ("B", "C", "theta"):
            d[k] = d[k][:, :, :groups].contiguous()
        if prev:
            d["B_prev"] = d["B_prev"][:, :groups].contiguous()
    return d


def _per_head(t, H, dim):
    return t if t is None or t.shape[dim] == H else t.repeat_interleave(H // t.shape[dim], dim=dim)


def _oracle(w, d, flags=0):
    H = w.nheads
    e = dict(d)
    for k in ("B", "C", "theta"):
        e[k] = _per_head(d[k], H, 2)
    e["B_prev"] = _per_head(d["B_prev"], H, 1)
    return oracle.scan(*(cpu64(e[k]) for k in ("x", "dt", "A", "lam", "theta", "B", "C", "h0",
                                                "x_prev", "B_prev")), flags=flags)


def _gpu(d, flags=0, out_dtype=torch.float32):
    g = {k: cuda(v) for k, v in d.items()}
    h = g["h0"].clone()
    y = m3.decode_tokens(h, g["x"], g["B"], g["C"], g["dt"], g["A"], g["lam"], g["theta"],
                         x_prev=g["x_prev"], B_prev=g["B_prev"], out_dtype=out_dtype, flags=flags)
    torch.cuda.synchronize()
    return y, h


def _check(w, d, flags=0, out_dtype=torch.float32, extra_tol=0.0):
    y, h = _gpu(d, flags, out_dtype)
    ref = _oracle(w, d, flags)
    ey, eh = rel_err(cpu64(y), ref.y), rel_err(cpu64(h), ref.hT)
    tol = TOL[w.torch_dtype]
    say(f"  y err {ey:.2e}  h err {eh:.2e}  (tol {tol:.0e})")
    assert ey <= tol + extra_tol and eh <= tol, (ey, eh)


@pytest.mark.parametrize("K", [1, 3, 16])
@pytest.mark.parametrize("R", [1, 4])
def test_tokens_bf16(K, R):
    w = I.Workload("t", 95, 3, K, 4, 64, 128, R, 64, "bf16")
    say(f"decode_tokens K={K} R={R}")
    _check(w, _inputs(w))


@pytest.mark.parametrize("P,N,R,dt", [
    (32, 64, 1, "bf16"), (64, 64, 1, "bf16"), (64, 64, 4, "bf16"), (16, 16, 1, "f32"),
    (64, 128, 1, "f32"), (32, 256, 1, "bf16"), (40, 64, 1, "bf16"), (32, 64, 2, "bf16"),
    (16, 32, 8, "bf16"), (48, 16, 3, "f32"), (64, 128, 4, "f32"),
    (80, 128, 1, "bf16"), (48, 256, 1, "f32"),   # rows of a unit split over blocks
    (16, 16, 4, "f32"), (48, 32, 4, "bf16"), (32, 64, 4, "f32"),   # rank 4: waves without rows
])
def test_tokens_shapes(P, N, R, dt):
    w = I.Workload("t", 96, 2, 5, 3, P, N, R, 64, dt)
    say(f"decode_tokens P={P} N={N} R={R} {dt}")
    _check(w, _inputs(w))


@pytest.mark.parametrize("P,N,R,dt", [
    (64, 64, 4, "bf16"), (32, 64, 2, "bf16"), (48, 16, 3, "f32"), (64, 128, 4, "f32"),
    (64, 128, 1, "f32"), (64, 64, 1, "bf16"), (16, 32, 2, "bf16"),
    (16, 16, 4, "f32"), (48, 32, 4, "bf16"),
])
def test_tokens_shapes_one_group(P, N, R, dt):
    """Calls of at most four tokens take kernels specialised for one group
    of tokens (single input with eight row passes, rank <= 4)."""
    w = I.Workload("t", 100, 2, 3, 3, P, N, R, 64, dt)
    say(f"decode_tokens one group P={P} N={N} R={R} {dt}")
    _check(w, _inputs(w))


@pytest.mark.parametrize("K", [4, 6])
@pytest.mark.parametrize("flags", [m3.M3_THETA_IS_ANGLE, m3.M3_A_PER_TOKEN])
@pytest.mark.parametrize("R", [1, 4])
def test_tokens_flags(flags, R, K):
    w = I.Workload("t", 97, 2, K, 3, 64, 128, R, 64, "bf16")
    d = _inputs(w)
    if flags & m3.M3_A_PER_TOKEN:
        rng = np.random.default_rng(7)
        d["A"] = torch.from_numpy(-np.exp(rng.uniform(-4, 0, size=(2, K, 3))).astype(np.float32))
    say(f"decode_tokens flags={flags} R={R} K={K}")
    _check(w, d, flags=flags)


@pytest.mark.parametrize("R", [1, 4])
def test_tokens_groups_no_prev_bf16_out(R):
    w = I.Workload("t", 98, 2, 4, 4, 64, 128, R, 64, "bf16")
    say(f"decode_tokens groups=2 R={R}")
    _check(w, _inputs(w, groups=2))
    say(f"decode_tokens no prev R={R}")
    _check(w, _inputs(w, prev=False))
    say(f"decode_tokens bf16 y R={R}")
    _check(w, _inputs(w), out_dtype=torch.bfloat16, extra_tol=2 ** -8)


@pytest.mark.parametrize("R", [1, 4])
def test_tokens_equal_single_steps(R):
    """K tokens in one call = K calls of m3_decode_step (GPU against GPU)."""
    K = 7
    w = I.Workload("t", 99, 2, K, 4, 64, 128, R, 64, "bf16")
    d = _inputs(w)
    y, h = _gpu(d)
    g = {k: cuda(v) for k, v in d.items()}
    hs = g["h0"].clone()
    ys = []
    for k in range(K):
        xp = g["x_prev"] if k == 0 else g["x"][:, k - 1].contiguous()
        Bp = g["B_prev"] if k == 0 else g["B"][:, k - 1].contiguous()
        ys.append(m3.decode_step(hs, g["x"][:, k].contiguous(), g["B"][:, k].contiguous(),
                                 g["C"][:, k].contiguous(), g["dt"][:, k].contiguous(), g["A"],
                                 g["lam"][:, k].contiguous(), g["theta"][:, k].contiguous(),
                                 x_prev=xp, B_prev=Bp))
    torch.cuda.synchronize()
    ey = rel_err(cpu64(y), cpu64(torch.stack(ys, dim=1)))
    eh = rel_err(cpu64(h), cpu64(hs))
    say(f"  tokens vs steps: y {ey:.2e}  h {eh:.2e}")
    assert ey <= 1e-5 and eh <= 1e-5, (ey, eh)


@pytest.mark.parametrize("name", ["siso_decode", "mimo_decode"])
def test_tokens_full_shape_sampled(name):
    """B=128, H=64, P=64, N=128, K=4 tokens in the benchmark's launch
    configuration; sampled batch rows against the oracle."""
    w = I.WORKLOADS[name].with_(seqlen=4)
    say(f"decode_tokens full shape {name}, K=4")
    d = _inputs(w)
    y, h = _gpu(d)
    rows = np.array([0, 77, 127])
    sub = {k: (v[rows] if v is not None and v.dim() > 1 else v) for k, v in d.items()}
    ref = _oracle(w.with_(batch=len(rows)), sub)
    ey, eh = rel_err(cpu64(y)[rows], ref.y), rel_err(cpu64(h)[rows], ref.hT)
    say(f"  y err {ey:.2e}  h err {eh:.2e}")
    assert ey <= 3e-3 and eh <= 3e-3, (ey, eh)


@pytest.mark.parametrize("R", [1, 4])
def test_tokens_deterministic_and_nan_stays_in_its_head(R):
    """Two calls on the same inputs agree bit for bit; a NaN in one head's x at
    token 2 (or in its B at token 1) reaches that head's state and its outputs
    from that token on, and nothing else (heads are independent and earlier
    outputs do not see it, also inside one group of four tokens)."""
    K = 4
    w = I.Workload("t", 96, 2, K, 4, 64, 128, R, 64, "bf16", "normal")
    d = _inputs(w)
    say(f"decode_tokens determinism and NaN isolation R={R}")
    y1, h1 = _gpu(d)
    y2, h2 = _gpu(d)
    assert torch.equal(y1.cpu(), y2.cpu()) and torch.equal(h1.cpu(), h2.cpu())
    x = d["x"].clone()
    x[1, 2, 3].view(-1)[5] = float("nan")
    y, h = _gpu(dict(d, x=x))
    bad_h = torch.isnan(h).flatten(2).any(dim=2).cpu()
    assert bad_h[1, 3] and bad_h.sum() == 1
    bad_y = torch.isnan(y).flatten(3).any(dim=3).cpu()          # [batch, token, head]
    expect = torch.zeros_like(bad_y)
    expect[1, 2:, 3] = True
    assert torch.equal(bad_y, expect)
    # a NaN in one head's B at token 1 reaches its outputs from token 1 on
    Bn = d["B"].clone()
    Bn[0, 1, 2].view(-1)[7] = float("nan")
    y, h = _gpu(dict(d, B=Bn))
    bad_h = torch.isnan(h).flatten(2).any(dim=2).cpu()
    assert bad_h[0, 2] and bad_h.sum() == 1
    bad_y = torch.isnan(y).flatten(3).any(dim=3).cpu()
    expect = torch.zeros_like(bad_y)
    expect[0, 1:, 2] = True
    assert torch.equal(bad_y, expect)
