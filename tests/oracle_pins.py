"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each ``check_*`` function runs the oracle library at ``lib`` on a small
seeded case and compares it with a formulation that does not go through the
oracle's sequential loop: a special case that reduces to a textbook
recurrence, the explicit complex-valued SSM, the real SSM with RoPE'd B/C,
an O(T^2) unrolled sum, a closed-form geometric series, the parity
state-tracking construction, second-order convergence of the trapezoid, and
MIMO as a sum of single-input runs.  They raise AssertionError on mismatch.

``tests/test_oracle_pins.py`` runs them on the real oracle; the mutation test
runs them on copies of the oracle with planted mistakes and requires each
mistake to be caught by at least one pin.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import oracle

TOL = 1e-11


def _rand_case(seed, Bsz=2, T=9, H=3, P=4, N=6, R=1, h0=True, prev=True):
    rng = np.random.default_rng(seed)
    d = dict(
        x=rng.standard_normal((Bsz, T, H, P, R)),
        dt=np.log1p(np.exp(rng.standard_normal((Bsz, T, H)))),
        A=-np.exp(rng.uniform(-4, 0, size=H)),
        lam=1 / (1 + np.exp(-rng.standard_normal((Bsz, T, H)))),
        theta=rng.uniform(-math.pi, math.pi, size=(Bsz, T, H, N // 2)),
        B=rng.standard_normal((Bsz, T, H, N, R)),
        C=rng.standard_normal((Bsz, T, H, N, R)),
        h0=rng.standard_normal((Bsz, H, P, N)) if h0 else None,
        x_prev=rng.standard_normal((Bsz, H, P, R)) if prev else None,
        B_prev=rng.standard_normal((Bsz, H, N, R)) if prev else None,
    )
    return d


def _scan(lib, d, flags=0):
    return oracle.scan(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"],
                       d.get("h0"), d.get("x_prev"), d.get("B_prev"), flags=flags,
                       lib_path=lib)


def _close(a, b, tol=TOL, what=""):
    err = float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0
    scale = max(1.0, float(np.max(np.abs(b)))) if np.size(b) else 1.0
    assert err <= tol * scale, f"{what}: max abs diff {err:.3e} (scale {scale:.2e})"
    return err


def _cplx(v, axis):
    """Real array with an even axis -> complex array over pairs (2k, 2k+1)."""
    v = np.moveaxis(v, axis, -1)
    c = v[..., 0::2] + 1j * v[..., 1::2]
    return np.moveaxis(c, -1, axis)


# ---------------------------------------------------------------------------
def check_euler_special_case(lib):
    """lam = 1 and theta = 0 leave the exponential-Euler (Mamba-2 style) rule
    h_t = exp(dt A) h_{t-1} + dt x_t B_t^T [xxxxx.co.kr Mamba-3 article,
    section 1.1: the earlier first-order rule that the trapezoid replaces]."""
    d = _rand_case(11, R=2)
    d["lam"] = np.ones_like(d["lam"])
    d["theta"] = np.zeros_like(d["theta"])
    got = _scan(lib, d)
    Bsz, T, H, P, R = d["x"].shape
    for b in range(Bsz):
        for h in range(H):
            S = d["h0"][b, h].copy()
            for t in range(T):
                S = math.exp(d["dt"][b, t, h] * d["A"][h]) * S \
                    + d["dt"][b, t, h] * d["x"][b, t, h] @ d["B"][b, t, h].T
                _close(got.y[b, t, h], S @ d["C"][b, t, h], what="euler y")
            _close(got.hT[b, h], S, what="euler hT")


def check_complex_form(lib, flags=0):
    """The complex-valued SSM written with complex numbers: N/2 complex
    states per row with transition z = exp(dt (A + i theta)) (or exp(dt A +
    i theta) when theta is the angle), b = B_even + i B_odd, and output
    Re(h conj(c)) [xxxxx.co.kr Mamba-3 article, section 1.2]."""
    d = _rand_case(12, R=2)
    got = _scan(lib, d, flags)
    Bsz, T, H, P, R = d["x"].shape
    for b in range(Bsz):
        for h in range(H):
            hc = _cplx(d["h0"][b, h], 1)
            xp, bp = d["x_prev"][b, h], _cplx(d["B_prev"][b, h], 0)
            for t in range(T):
                dt, lam = d["dt"][b, t, h], d["lam"][b, t, h]
                th = d["theta"][b, t, h]
                ang = th if (flags & oracle.THETA_IS_ANGLE) else dt * th
                z = np.exp(dt * d["A"][h] + 1j * ang)            # [N/2]
                bt = _cplx(d["B"][b, t, h], 0)                    # [N/2, R]
                ct = _cplx(d["C"][b, t, h], 0)
                xt = d["x"][b, t, h]                              # [P, R]
                hc = z[None, :] * hc + (1 - lam) * dt * z[None, :] * (xp @ bp.T) \
                    + lam * dt * (xt @ bt.T)
                y = np.real(hc @ np.conj(ct))                     # [P, R]
                _close(got.y[b, t, h], y, what="complex y")
                xp, bp = xt, bt
            hr = np.empty_like(d["h0"][b, h])
            hr[:, 0::2], hr[:, 1::2] = hc.real, hc.imag
            _close(got.hT[b, h], hr, what="complex hT")


def _rot(v, ang):
    """Rotate pairs (2k, 2k+1) along the last-but-R axis convention used here:
    v [..., N] with ang [N/2] -> each pair rotated by +ang."""
    c, s = np.cos(ang), np.sin(ang)
    out = np.empty_like(v)
    out[..., 0::2] = c * v[..., 0::2] - s * v[..., 1::2]
    out[..., 1::2] = s * v[..., 0::2] + c * v[..., 1::2]
    return out


def check_rope_frame(lib):
    """The "RoPE trick": the same outputs from a real SSM with no rotation in
    its transition, whose B and C are rotated by minus the cumulative angle
    Phi_t = sum_{r<=t} dt_r theta_r; the true state is the rotated-back
    frame state [xxxxx.co.kr Mamba-3 article, section 1.2]."""
    d = _rand_case(13, R=3)
    got = _scan(lib, d)
    Bsz, T, H, P, R = d["x"].shape
    for b in range(Bsz):
        for h in range(H):
            Phi = np.zeros(d["theta"].shape[-1])
            Ht = d["h0"][b, h].copy()            # frame state, Phi_{-1} = 0
            xp = d["x_prev"][b, h]
            bpt = d["B_prev"][b, h]              # rotated by -Phi_{-1} = 0
            for t in range(T):
                dt, lam = d["dt"][b, t, h], d["lam"][b, t, h]
                Phi = Phi + dt * d["theta"][b, t, h]
                Bt = _rot(d["B"][b, t, h].T, -Phi).T       # [N, R]
                Ct = _rot(d["C"][b, t, h].T, -Phi).T
                al = math.exp(dt * d["A"][h])
                Ht = al * Ht + (1 - lam) * dt * al * (xp @ bpt.T) \
                    + lam * dt * (d["x"][b, t, h] @ Bt.T)
                _close(got.y[b, t, h], Ht @ Ct, what="rope y")
                xp, bpt = d["x"][b, t, h], Bt
            _close(got.hT[b, h], _rot(Ht, Phi), what="rope hT")


def check_unrolled(lib):
    """Brute-force O(T^2) unrolled sum (T <= 8): every output is the decayed,
    rotated sum over all earlier inputs with the trapezoid weights
      w_{t,s} = lam_s dt_s + [s < t] (1 - lam_{s+1}) dt_{s+1},
    plus the initial state and the token before the first one."""
    d = _rand_case(14, T=8, R=2)
    got = _scan(lib, d)
    Bsz, T, H, P, R = d["x"].shape
    for b in range(Bsz):
        for h in range(H):
            dt, lam = d["dt"][b, :, h], d["lam"][b, :, h]
            cs = np.cumsum(dt * d["A"][h])
            Phi = np.cumsum(dt[:, None] * d["theta"][b, :, h], axis=0)
            for t in range(T):
                S = math.exp(cs[t]) * _rot(d["h0"][b, h], Phi[t])
                S = S + math.exp(cs[t]) * (1 - lam[0]) * dt[0] * _rot(
                    d["x_prev"][b, h] @ d["B_prev"][b, h].T, Phi[t])
                for s in range(t + 1):
                    w = lam[s] * dt[s] + ((1 - lam[s + 1]) * dt[s + 1] if s < t else 0.0)
                    u = d["x"][b, s, h] @ d["B"][b, s, h].T
                    S = S + math.exp(cs[t] - cs[s]) * w * _rot(u, Phi[t] - Phi[s])
                _close(got.y[b, t, h], S @ d["C"][b, t, h], what="unrolled y")
                if t == T - 1:
                    _close(got.hT[b, h], S, what="unrolled hT")


def check_closed_form(lib):
    """Constant dt, A, lam, theta, x and B: the state is a geometric series,
      h_{T-1} = z^T h0 + z^{T-1} g u + (b' z + g) u (1 - z^{T-1}) / (1 - z)
    with z = exp(dt (A + i theta)) per pair, u = x b^T, g = lam dt and
    b' = (1 - lam) dt (no token before the first)."""
    rng = np.random.default_rng(15)
    T, H, P, N, R = 37, 2, 3, 8, 2
    dt0, lam0 = 0.7, 0.35
    A = np.array([-0.3, -0.05])
    th0 = rng.uniform(-math.pi, math.pi, size=(H, N // 2))
    x0 = rng.standard_normal((H, P, R))
    B0 = rng.standard_normal((H, N, R))
    C0 = rng.standard_normal((H, N, R))
    h0 = rng.standard_normal((1, H, P, N))
    d = dict(x=np.broadcast_to(x0, (1, T, H, P, R)), dt=np.full((1, T, H), dt0),
             A=A, lam=np.full((1, T, H), lam0),
             theta=np.broadcast_to(th0, (1, T, H, N // 2)),
             B=np.broadcast_to(B0, (1, T, H, N, R)), C=np.broadcast_to(C0, (1, T, H, N, R)),
             h0=h0)
    got = _scan(lib, d)
    for h in range(H):
        z = np.exp(dt0 * A[h] + 1j * dt0 * th0[h])[None, :]
        u = x0[h] @ _cplx(B0[h], 0).T
        g, bp = lam0 * dt0, (1 - lam0) * dt0
        hc = z ** T * _cplx(h0[0, h], 1) + z ** (T - 1) * g * u \
            + (bp * z + g) * u * (1 - z ** (T - 1)) / (1 - z)
        y = np.real(hc @ np.conj(_cplx(C0[h], 0)))
        _close(got.y[0, T - 1, h], y, tol=1e-10, what="closed-form y")
        hr = np.empty((P, N))
        hr[:, 0::2], hr[:, 1::2] = hc.real, hc.imag
        _close(got.hT[0, h], hr, tol=1e-10, what="closed-form hT")


def parity_case(bits):
    """Parity by rotation [no1joon.github.io Mamba-3 review, section on the
    paper's three answers (complex state, parity of a bit string);
    xxxxx.co.kr Mamba-3 article, section 1.2].  One complex pair, no decay
    (A = 0), lam = 1, dt = 1, theta_t = pi * bit_t and a single unit input at
    t = 0: each 1-bit turns the state by pi, so y_t = +-1 gives the parity of
    bits 1..t (bit 0 arrives with the input, which is not rotated)."""
    T = len(bits)
    d = dict(x=np.zeros((1, T, 1, 1, 1)), dt=np.ones((1, T, 1)), A=np.zeros(1),
             lam=np.ones((1, T, 1)),
             theta=(math.pi * np.asarray(bits, float)).reshape(1, T, 1, 1),
             B=np.zeros((1, T, 1, 2, 1)), C=np.zeros((1, T, 1, 2, 1)))
    d["x"][0, 0] = 1.0
    d["B"][..., 0, 0] = 1.0
    d["C"][..., 0, 0] = 1.0
    return d


def check_parity(lib, bits=None):
    if bits is None:
        bits = np.random.default_rng(16).integers(0, 2, size=40)
    got = _scan(lib, parity_case(bits))
    y = got.y[0, :, 0, 0, 0]
    expect = np.array([(-1.0) ** (int(np.sum(bits[1:t + 1])) % 2) for t in range(len(bits))])
    _close(y, expect, tol=1e-9, what="parity")


def _ode_error(lib, n, lam_v, a=-0.8, w=2.3, b=(0.7, -0.4), tend=1.0):
    """Integrate h' = (a + i w) h + b u(s), u(s) = cos(3 s) + 0.5, h(0)=0.3+0.1i
    over [0, tend] with n steps of the recurrence; return |h_n - h(tend)|."""
    from scipy.integrate import quad
    lam_c = complex(a, w)
    bc = complex(*b)
    u = lambda s: math.cos(3 * s) + 0.5
    h_init = complex(0.3, 0.1)
    re = quad(lambda s: (np.exp(lam_c * (tend - s)) * bc * u(s)).real, 0, tend,
              epsabs=1e-14, epsrel=1e-14, limit=200)[0]
    im = quad(lambda s: (np.exp(lam_c * (tend - s)) * bc * u(s)).imag, 0, tend,
              epsabs=1e-14, epsrel=1e-14, limit=200)[0]
    exact = np.exp(lam_c * tend) * h_init + complex(re, im)
    step = tend / n
    grid = np.arange(n + 1) * step
    d = dict(x=np.array([u(s) for s in grid[1:]]).reshape(1, n, 1, 1, 1),
             dt=np.full((1, n, 1), step), A=np.array([a]), lam=np.full((1, n, 1), lam_v),
             theta=np.full((1, n, 1, 1), w),
             B=np.broadcast_to(np.array(b).reshape(1, 1, 1, 2, 1), (1, n, 1, 2, 1)),
             C=np.zeros((1, n, 1, 2, 1)),
             h0=np.array([[[[h_init.real, h_init.imag]]]]),
             x_prev=np.array([[[[u(0.0)]]]]), B_prev=np.array(b).reshape(1, 1, 2, 1))
    got = _scan(lib, d)
    return abs(complex(got.hT[0, 0, 0, 0], got.hT[0, 0, 0, 1]) - exact)


def check_second_order(lib):
    """The exponential-trapezoidal rule approximates the state-input integral
    to second order, the exponential-Euler rule to first order
    [xxxxx.co.kr Mamba-3 article, section 1.1].  With lam = 1/2 the error
    falls ~4x when the step halves; with lam = 1 ~2x."""
    e_tr = [_ode_error(lib, n, 0.5) for n in (64, 128, 256)]
    e_eu = [_ode_error(lib, n, 1.0) for n in (64, 128, 256)]
    r_tr = [e_tr[i] / e_tr[i + 1] for i in range(2)]
    r_eu = [e_eu[i] / e_eu[i + 1] for i in range(2)]
    assert all(3.6 < r < 4.4 for r in r_tr), f"trapezoid ratios {r_tr}"
    assert all(1.8 < r < 2.2 for r in r_eu), f"euler ratios {r_eu}"
    return r_tr, r_eu


def check_mimo_sum_of_siso(lib):
    """MIMO uses the single-input recurrence as a black box [velog.io Mamba3
    review, introduction]: column r' of the rank-R output is the sum over r
    of single-input runs on (x[:, r], B[:, r]) read out with C[:, r']; the
    initial state goes into one of them."""
    d = _rand_case(17, R=3)
    got = _scan(lib, d)
    R = d["x"].shape[-1]
    y = np.zeros_like(got.y)
    hT = np.zeros_like(got.hT)
    for r in range(R):
        for rr in range(R):
            sub = dict(d)
            sub["x"] = d["x"][..., r:r + 1]
            sub["B"] = d["B"][..., r:r + 1]
            sub["C"] = d["C"][..., rr:rr + 1]
            sub["x_prev"] = d["x_prev"][..., r:r + 1]
            sub["B_prev"] = d["B_prev"][..., r:r + 1]
            sub["h0"] = d["h0"] if r == 0 else np.zeros_like(d["h0"])
            res = _scan(lib, sub)
            y[..., rr:rr + 1] += res.y
            if rr == 0:
                hT += res.hT
    _close(got.y, y, what="mimo y")
    _close(got.hT, hT, what="mimo hT")


def check_split_and_decode(lib):
    """A scan split in two, the second part given the first part's final
    state and last token as (h0, x_prev, B_prev), equals the whole scan; a
    decode step after a scan of T-1 tokens equals the scan of T tokens."""
    d = _rand_case(18, T=11, R=2)
    whole = _scan(lib, d)
    k = 5
    first = dict(d, x=d["x"][:, :k], dt=d["dt"][:, :k], lam=d["lam"][:, :k],
                 theta=d["theta"][:, :k], B=d["B"][:, :k], C=d["C"][:, :k])
    r1 = _scan(lib, first)
    second = dict(d, x=d["x"][:, k:], dt=d["dt"][:, k:], lam=d["lam"][:, k:],
                  theta=d["theta"][:, k:], B=d["B"][:, k:], C=d["C"][:, k:],
                  h0=r1.hT, x_prev=d["x"][:, k - 1], B_prev=d["B"][:, k - 1])
    r2 = _scan(lib, second)
    _close(np.concatenate([r1.y, r2.y], axis=1), whole.y, tol=1e-13, what="split y")
    _close(r2.hT, whole.hT, tol=1e-13, what="split hT")
    T = d["x"].shape[1]
    head = dict(d, x=d["x"][:, :T - 1], dt=d["dt"][:, :T - 1], lam=d["lam"][:, :T - 1],
                theta=d["theta"][:, :T - 1], B=d["B"][:, :T - 1], C=d["C"][:, :T - 1])
    rh = _scan(lib, head)
    y, hn = oracle.decode_step(rh.hT, d["x"][:, T - 1], d["x"][:, T - 2], d["B"][:, T - 1],
                               d["B"][:, T - 2], d["C"][:, T - 1], d["dt"][:, T - 1],
                               d["A"], d["lam"][:, T - 1], d["theta"][:, T - 1],
                               lib_path=lib)
    _close(y, whole.y[:, T - 1], tol=1e-13, what="decode y")
    _close(hn, whole.hT, tol=1e-13, what="decode h")


def check_linearity_and_independence(lib):
    """The map (x, h0, x_prev) -> (y, hT) is linear for fixed dt, A, lam,
    theta, B, C; and each (batch, head) pair evolves on its own."""
    d = _rand_case(19, R=2)
    e = _rand_case(20, R=2)
    mix = dict(d, x=2.0 * d["x"] - 0.5 * e["x"], h0=2.0 * d["h0"] - 0.5 * e["h0"],
               x_prev=2.0 * d["x_prev"] - 0.5 * e["x_prev"])
    e2 = dict(d, x=e["x"], h0=e["h0"], x_prev=e["x_prev"])
    rd, re_, rm = _scan(lib, d), _scan(lib, e2), _scan(lib, mix)
    _close(rm.y, 2.0 * rd.y - 0.5 * re_.y, tol=1e-12, what="linear y")
    _close(rm.hT, 2.0 * rd.hT - 0.5 * re_.hT, tol=1e-12, what="linear hT")
    h = 1
    sl = dict(d, x=d["x"][:, :, h:h + 1], dt=d["dt"][:, :, h:h + 1], A=d["A"][h:h + 1],
              lam=d["lam"][:, :, h:h + 1], theta=d["theta"][:, :, h:h + 1],
              B=d["B"][:, :, h:h + 1], C=d["C"][:, :, h:h + 1], h0=d["h0"][:, h:h + 1],
              x_prev=d["x_prev"][:, h:h + 1], B_prev=d["B_prev"][:, h:h + 1])
    rs = _scan(lib, sl)
    _close(rs.y, rd.y[:, :, h:h + 1], tol=0.0, what="head slice y")
    _close(rs.hT, rd.hT[:, h:h + 1], tol=0.0, what="head slice hT")


def _complex_token(hc, xp, bp, xt, bt, ct, dt, a, lam, ang):
    """One token of the complex-valued SSM in complex numbers (see
    check_complex_form): hc [P, N/2] complex, bp/bt/ct [N/2, R] complex."""
    z = np.exp(dt * a + 1j * ang)
    hc = z[None, :] * hc + lam * dt * (xt @ bt.T)
    if xp is not None:
        hc = hc + (1 - lam) * dt * z[None, :] * (xp @ bp.T)
    return hc, np.real(hc @ np.conj(ct))


def check_a_per_token(lib):
    """A_t drawn independently for every (batch, token, head) [xxxxx.co.kr
    Mamba-3 article, section 1.1 writes the decay as exp(dt_t A_t)]: the
    scan with the per-token flag against the complex-valued SSM evaluated
    with that token's own A; then one decode step with A drawn per (batch,
    head) against one complex token from the same state."""
    d = _rand_case(21, R=2)
    rng = np.random.default_rng(22)
    Bsz, T, H, P, R = d["x"].shape
    d["A"] = -np.exp(rng.uniform(-4, 0.5, size=(Bsz, T, H)))
    got = _scan(lib, d, flags=oracle.A_PER_TOKEN)
    for b in range(Bsz):
        for h in range(H):
            hc = _cplx(d["h0"][b, h], 1)
            xp, bp = d["x_prev"][b, h], _cplx(d["B_prev"][b, h], 0)
            for t in range(T):
                dt = d["dt"][b, t, h]
                xt, bt = d["x"][b, t, h], _cplx(d["B"][b, t, h], 0)
                hc, y = _complex_token(hc, xp, bp, xt, bt, _cplx(d["C"][b, t, h], 0), dt,
                                       d["A"][b, t, h], d["lam"][b, t, h],
                                       dt * d["theta"][b, t, h])
                _close(got.y[b, t, h], y, what="A per token y")
                xp, bp = xt, bt
            hr = np.empty((P, hc.shape[1] * 2))
            hr[:, 0::2], hr[:, 1::2] = hc.real, hc.imag
            _close(got.hT[b, h], hr, what="A per token hT")
    # decode step: A [Bsz, H], one value per (batch, head)
    A2 = -np.exp(rng.uniform(-4, 0.5, size=(Bsz, H)))
    t = 3
    y, hn = oracle.decode_step(d["h0"], d["x"][:, t], d["x"][:, t - 1], d["B"][:, t],
                               d["B"][:, t - 1], d["C"][:, t], d["dt"][:, t], A2,
                               d["lam"][:, t], d["theta"][:, t], flags=oracle.A_PER_TOKEN,
                               lib_path=lib)
    for b in range(Bsz):
        for h in range(H):
            dt = d["dt"][b, t, h]
            hc, yc = _complex_token(_cplx(d["h0"][b, h], 1), d["x"][b, t - 1, h],
                                    _cplx(d["B"][b, t - 1, h], 0), d["x"][b, t, h],
                                    _cplx(d["B"][b, t, h], 0), _cplx(d["C"][b, t, h], 0), dt,
                                    A2[b, h], d["lam"][b, t, h], dt * d["theta"][b, t, h])
            _close(y[b, h], yc, what="decode A per (batch, head) y")
            _close(hn[b, h, :, 0::2], hc.real, what="decode A per (batch, head) h")
            _close(hn[b, h, :, 1::2], hc.imag, what="decode A per (batch, head) h")


# ---------------------------------------------------------------------------
# gradients: central finite differences of the forward scan
def _loss(lib, d, dy, dhT, flags):
    r = _scan(lib, d, flags)
    return float(np.sum(r.y * dy) + (np.sum(r.hT * dhT) if dhT is not None else 0.0))


def _fd_case(lib, seed, flags=0, R=1, h0=True, prev=True, with_dhT=True, tol=1e-7):
    """Each gradient's inner product with a random direction against
    (L(p + e v) - L(p - e v)) / 2e, L = <y, dy> + <hT, dhT>, in fp64."""
    d = _rand_case(seed, Bsz=2, T=7, H=2, P=3, N=4, R=R, h0=h0, prev=prev)
    rng = np.random.default_rng(seed + 1000)
    if flags & oracle.A_PER_TOKEN:
        d["A"] = -np.exp(rng.uniform(-4, 0, size=d["dt"].shape))
    dy = rng.standard_normal(d["x"].shape)
    dhT = rng.standard_normal((2, 2, 3, 4)) if with_dhT else None
    g = oracle.scan_backward(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"],
                             d["h0"], d["x_prev"], d["B_prev"], dy, dhT, flags=flags, lib_path=lib)
    eps = 1e-6
    for name in oracle.GRAD_NAMES:
        if d.get(name) is None:
            assert g[name] is None, name
            continue
        v = rng.standard_normal(d[name].shape)
        dp = dict(d)
        dp[name] = d[name] + eps * v
        dm = dict(d)
        dm[name] = d[name] - eps * v
        fd = (_loss(lib, dp, dy, dhT, flags) - _loss(lib, dm, dy, dhT, flags)) / (2 * eps)
        an = float(np.sum(g[name] * v))
        assert abs(fd - an) <= tol * max(1.0, abs(fd)), f"d{name}: analytic {an:.10e} vs fd {fd:.10e}"


def check_backward_siso(lib):
    """Gradients of the single-input scan, with h0, the token before and dhT."""
    _fd_case(lib, 40, R=1)


def check_backward_mimo_and_flags(lib):
    """Rank 3; theta as the angle itself; A per token; no h0 / previous
    token / dhT."""
    _fd_case(lib, 41, R=3)
    _fd_case(lib, 42, flags=oracle.THETA_IS_ANGLE, R=2)
    _fd_case(lib, 43, flags=oracle.A_PER_TOKEN, R=1)
    _fd_case(lib, 44, R=2, h0=False, prev=False, with_dhT=False)


# ---------------------------------------------------------------------------
# B/C preparation (RMS normalisation, weight, per-head bias)
def _bc_case(seed, rows=3, G=2, H=4, N=8, R=3):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((rows, G, N, R)) * rng.uniform(0.2, 5.0, size=(rows, G, 1, R))
    w = rng.uniform(0.5, 2.0, size=N)
    bias = rng.standard_normal((H, N, R)) * 3.0
    return v, w, bias


def check_bc_prep_unit_rms(lib):
    """With weight 1, no bias and eps 0, every (row, head, rank column) comes
    out with mean square exactly 1 over N, as a positive multiple of its input
    column: what an RMS normalisation over the state channels is."""
    v, _, _ = _bc_case(30)
    out = oracle.bc_prep(v, 4, eps=0.0, lib_path=lib)
    _close(np.mean(out ** 2, axis=-2), np.ones(out.shape[:-2] + out.shape[-1:]), tol=1e-13,
           what="mean square over N")
    vg = np.repeat(v, 2, axis=1)                      # group g serves heads 2g, 2g + 1
    ratio = out / vg
    assert np.all(ratio > 0), "direction of the column"
    _close(ratio, np.broadcast_to(ratio[..., :1, :], ratio.shape), tol=1e-13, what="one factor per column")


def check_bc_prep_scale_invariance(lib):
    """Scaling one rank column of one token by c > 0 changes nothing (eps 0):
    the normalisation runs per column, not over the whole N x R block."""
    v, w, bias = _bc_case(31)
    base = oracle.bc_prep(v, 4, w, bias, eps=0.0, lib_path=lib)
    v2 = v.copy()
    v2[1, 0, :, 2] *= 7.5
    v2[2, 1, :, 0] *= 0.01
    _close(oracle.bc_prep(v2, 4, w, bias, eps=0.0, lib_path=lib), base, tol=1e-13,
           what="per-column scale invariance")


def check_bc_prep_bias_weight_eps(lib):
    """Zero input columns come out as exactly the bias of each head (heads
    of one group get their own bias, added after the normalisation); an input
    c u with u of unit mean square comes out as w c u / sqrt(c^2 + eps) plus
    the bias (the closed form of the normalisation with eps)."""
    v, w, bias = _bc_case(32)
    z = np.zeros_like(v)
    _close(oracle.bc_prep(z, 4, w, bias, eps=1e-3, lib_path=lib),
           np.broadcast_to(bias, (3, 4, 8, 3)), tol=0.0, what="zero input gives the head's bias")
    u = v / np.sqrt(np.mean(v ** 2, axis=-2, keepdims=True))
    c, eps = 0.3, 0.05
    got = oracle.bc_prep(c * u, 4, w, bias, eps=eps, lib_path=lib)
    ug = np.repeat(u, 2, axis=1)
    want = w[:, None] * c * ug / math.sqrt(c * c + eps) + bias
    _close(got, want, tol=1e-13, what="closed form with eps")
    # without the normalisation only the weight and bias act
    _close(oracle.bc_prep(v, 4, w, None, rms=False, lib_path=lib),
           w[:, None] * np.repeat(v, 2, axis=1), tol=0.0, what="weight alone")


# ---------------------------------------------------------------------------
# angle projection (theta from the layer input)
def check_theta_proj_columns_and_linearity(lib):
    """A linear map per head group is fixed by its response to the unit
    inputs (column j of each group's matrix) and by linearity; a zero input
    gives zero angles."""
    rng = np.random.default_rng(40)
    G, K, D = 3, 5, 7
    W = rng.standard_normal((G, K, D))
    eye = np.eye(D)
    got = oracle.theta_proj(eye, W, lib_path=lib)            # [D, G, K]
    for j in range(D):
        _close(got[j], W[:, :, j], tol=0.0, what=f"unit input {j}")
    u1, u2 = rng.standard_normal((4, D)), rng.standard_normal((4, D))
    a = oracle.theta_proj(2.5 * u1 - 0.75 * u2, W, lib_path=lib)
    b = 2.5 * oracle.theta_proj(u1, W, lib_path=lib) - 0.75 * oracle.theta_proj(u2, W, lib_path=lib)
    _close(a, b, tol=1e-13, what="linearity")
    _close(oracle.theta_proj(np.zeros((2, D)), W, lib_path=lib), np.zeros((2, G, K)), tol=0.0,
           what="zero input")


def check_theta_proj_parity(lib):
    """The parity construction [no1joon.github.io Mamba-3 review, the paper's
    three answers; xxxxx.co.kr Mamba-3 article, section 1.2] with its angles
    produced by the projection: u_t = (bit_t, noise) and a group matrix that
    reads pi times the first input only, so the scan still tracks parity."""
    bits = np.random.default_rng(41).integers(0, 2, size=24)
    d = parity_case(bits)
    T = len(bits)
    rng = np.random.default_rng(42)
    u = np.stack([bits.astype(float), rng.standard_normal(T), rng.standard_normal(T)], axis=-1)
    W = np.array([[[math.pi, 0.0, 0.0]]])                     # G = 1, K = 1, D = 3
    d["theta"] = oracle.theta_proj(u.reshape(1, T, 3), W, lib_path=lib)   # [1, T, 1, 1]
    got = _scan(lib, d)
    y = got.y[0, :, 0, 0, 0]
    expect = np.array([(-1.0) ** (int(np.sum(bits[1:t + 1])) % 2) for t in range(T)])
    _close(y, expect, tol=1e-9, what="parity through the projection")


ALL_CHECKS = [check_euler_special_case, check_complex_form, check_rope_frame,
              check_unrolled, check_closed_form, check_parity, check_second_order,
              check_mimo_sum_of_siso, check_split_and_decode,
              check_linearity_and_independence, check_a_per_token, check_bc_prep_unit_rms,
              check_bc_prep_scale_invariance, check_bc_prep_bias_weight_eps, check_backward_siso,
              check_backward_mimo_and_flags, check_theta_proj_columns_and_linearity,
              check_theta_proj_parity]
