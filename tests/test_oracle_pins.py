"""Host-only pins of the fp64 oracle (no GPU)."""
import os
import re
import tempfile

import numpy as np
import pytest

from oracle import oracle
from tests import oracle_pins as pins

LIB = oracle.load() and oracle._LIB


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check(LIB)


def test_complex_form_theta_is_angle():
    pins.check_complex_form(LIB, flags=oracle.THETA_IS_ANGLE)


def test_second_order_ratios():
    r_tr, r_eu = pins.check_second_order(LIB)
    assert min(r_tr) > max(r_eu) + 1.0


def test_parity_all_short_strings():
    # every bit string of length 8: the sign tracks the parity exactly
    for v in range(256):
        bits = np.array([(v >> i) & 1 for i in range(8)])
        pins.check_parity(LIB, bits)


def test_real_eigenvalues_cannot_track_parity():
    # with the rotation switched off (theta = 0) the output is the same for
    # every bit string: a real-only transition carries no parity
    d = pins.parity_case(np.array([0, 1, 1, 0, 1, 0, 0, 1]))
    d["theta"] = np.zeros_like(d["theta"])
    y = oracle.scan(d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"]).y
    assert np.all(y[0, :, 0, 0, 0] == 1.0)


def test_golden_notebook_state_size():
    """The notebook measurement on the no1joon.github.io Mamba-3 review
    (section on measuring it directly) lists a recurrent state of 0.25 MiB
    per layer at every length from 1,024 to 65,536 tokens, for fp16, d_model
    1024, 16 heads and state size 128 (head dim 1024/16 = 64).  The oracle's
    final state [Bsz, H, P, N] has exactly that size and does not grow with T."""
    path = os.path.join(os.path.dirname(__file__), "golden", "notebook_state_size.txt")
    rows = [ln.split() for ln in open(path) if ln.strip() and not ln.startswith("#")]
    H, P, N = 16, 1024 // 16, 128
    for length, kv_mib, state_mib in rows:
        length = int(length)
        # the state after a scan of `length` tokens: shape is independent of T;
        # run a short scan with the same (H, P, N) to read the shape
        T = 2
        zeros = np.zeros
        res = oracle.scan(zeros((1, T, H, P, 1)), np.ones((1, T, H)), -np.ones(H),
                          np.ones((1, T, H)) * 0.5, zeros((1, T, H, N // 2)),
                          zeros((1, T, H, N, 1)), zeros((1, T, H, N, 1)))
        assert res.hT.shape == (1, H, P, N)
        assert res.hT.size * 2 / 2 ** 20 == float(state_mib)
        # the attention cache in the same table grows linearly with length:
        # K and V, 2 bytes each, d_model 1024 per token
        assert 2 * 2 * 1024 * length / 2 ** 20 == float(kv_mib)


# ---------------------------------------------------------------------------
# Planted mistakes: each mutant of the oracle source must fail some pin.
MUTANTS = {
    "drop_beta_term": ("s += beta * u;", "s += 0.0 * u;"),
    "beta_without_one_minus_lam": ("(1.0 - lam) * dt * alpha", "lam * dt * alpha"),
    "beta_without_alpha": ("(1.0 - lam) * dt * alpha", "(1.0 - lam) * dt"),
    "gamma_with_alpha": ("const double gamma = lam * dt;", "const double gamma = lam * dt * alpha;"),
    "prev_uses_current_x": ("u += xp[p * R + r] * bp[n * R + r];", "u += x[p * R + r] * bp[n * R + r];"),
    "rotation_sign": ("cs * re - sn * im;", "cs * re + sn * im;"),
    "phase_without_dt": (": dt * theta[k];", ": theta[k];"),
    "output_reads_B": ("acc += S[p * N + n] * c[n * R + r];", "acc += S[p * N + n] * b[n * R + r];"),
    "mimo_transposed_index": ("u += x[p * R + r] * b[n * R + r];", "u += x[p * R + r] * b[r * N + n];"),
    "pair_index_swapped": ("const double re = S[p * N + 2 * k], im = S[p * N + 2 * k + 1];",
                           "const double im = S[p * N + 2 * k], re = S[p * N + 2 * k + 1];"),
    "decay_sign": ("exp(dt * A)", "exp(-dt * A)"),
    "prev_not_advanced": ("      xp = xt;\n      bp = bt;\n", "\n"),
    "bc_sum_not_mean": ("sqrt(ms / (double)N + eps)", "sqrt(ms + eps)"),
    "bc_eps_outside_sqrt": ("1.0 / sqrt(ms / (double)N + eps)", "1.0 / (sqrt(ms / (double)N) + eps)"),
    "bc_bias_by_group": ("bias[(h * N + n) * R + r]", "bias[(g * N + n) * R + r]"),
    "bc_bias_inside_norm": ("wn * v[n * R + r] * scale + bn;", "wn * (v[n * R + r] + bn) * scale;"),
    "bc_weight_by_rank": ("w ? w[n] : 1.0", "w ? w[r] : 1.0"),
    "bwd_rotation_derivative_sign": ("dphi += -g0 * w1 + g1 * w0;", "dphi += g0 * w1 - g1 * w0;"),
    "bwd_adjoint_rotation_sign": ("V[p * N + 2 * k] = cs * g0 + sn * g1;", "V[p * N + 2 * k] = cs * g0 - sn * g1;"),
    "bwd_state_gradient_without_decay": ("G[i] = alpha * V[i];", "G[i] = V[i];"),
    "bwd_beta_chain_without_decay_term": ("(1.0 - LM) * alpha * (1.0 + DT * AA) * dbeta", "(1.0 - LM) * alpha * dbeta"),
    "bwd_theta_without_dt": ("dtheta[bth * K + k] = angle ? dphi : DT * dphi;", "dtheta[bth * K + k] = dphi;"),
    "bwd_output_grad_skipped": ("G[p * N + n] += v;", "G[p * N + n] += 0.0 * v;"),
    "bwd_prev_x_uses_gamma": ("gx[t * P * R + p * R + r] += beta * v;", "gx[t * P * R + p * R + r] += gamma * v;"),
    "scan_a_per_token_read_per_head": ("const double a = (d->flags & M3REF_A_PER_TOKEN) ? A[bth] : A[h];",
                                       "const double a = (d->flags & M3REF_A_PER_TOKEN) ? A[h] : A[h];"),
    "decode_a_per_token_read_per_head": ("const double a = (d->flags & M3REF_A_PER_TOKEN) ? A[u] : A[h_];",
                                         "const double a = (d->flags & M3REF_A_PER_TOKEN) ? A[h_] : A[h_];"),
    "theta_proj_transposed": ("W[(g * K + k) * D + j]", "W[(g * D + j) * K + k]"),
    "theta_proj_group_ignored": ("out[(i * G + g) * K + k] = acc;", "out[(i * G + g) * K + k] = g ? 0.0 : acc;"),
    "theta_proj_last_input_dropped": ("for (int64_t j = 0; j < D; ++j) acc +=", "for (int64_t j = 0; j < D - 1; ++j) acc +="),
    "bc_norm_over_all_ranks": ("for (int64_t n = 0; n < N; ++n) ms += v[n * R + r] * v[n * R + r];",
                               "for (int64_t n = 0; n < N * R; ++n) ms += v[n] * v[n];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle._SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mutated = src.replace(old, new)
    msrc = tmp_path / "m3_oracle_mutant.c"
    msrc.write_text(mutated)
    lib = str(tmp_path / "libmutant.so")
    oracle.build(src=str(msrc), out=lib, extra=("-w",))
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            check(lib)
        except AssertionError as exc:  # the pin caught the mistake
            caught.append((check.__name__, str(exc)[:80]))
    assert caught, f"mutant {name} passed every pin"
