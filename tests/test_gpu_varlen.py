"""GPU parity of m3_scan_prefill_varlen (sequences packed back to back)
against the fp64 oracle run on each sequence alone, and against one
m3_scan_prefill call per sequence (GPU against GPU, bit for bit)."""
import numpy as np
import pytest
import torch

from linear_recurrent_sequence_mamba_amd import binding as m3
from linear_recurrent_sequence_mamba_amd import inputs as I
from oracle import oracle
from tests.util import TOL, cpu64, cuda, rel_err, say

pytestmark = pytest.mark.gpu

TOK = ("x", "dt", "lam", "theta", "B", "C")
SEQ = ("h0", "x_prev", "B_prev")

# empty sequences, one token, exactly one chunk, one chunk plus one token,
# several chunks with ragged tails
LENGTHS = [0, 1, 63, 64, 65, 130, 200, 0, 7]


def _packed(w, lengths, groups=None, prev=True, h0="normal"):
    d = I.packed_inputs(w.with_(batch=1, seqlen=sum(lengths)), lengths, h0=h0, with_prev=prev)
    if groups is not None:
        for k in ("B", "C", "theta"):
            d[k] = d[k][:, :groups].contiguous()
        if prev:
            d["B_prev"] = d["B_prev"][:, :groups].contiguous()
    return d


def _cu(d):
    return [int(v) for v in d["cu_seqlens"]]


def _run_varlen(d, flags=0, out_dtype=torch.float32, y_fill=None):
    g = {k: cuda(v) for k, v in d.items()}
    T, H, P, R = d["x"].shape
    S = len(d["cu_seqlens"]) - 1
    G, N = d["B"].shape[1], d["B"].shape[2]
    dims = m3.make_dims(S, T, H, P, N, R, 0, m3.dtype_code(d["x"].dtype), m3.dtype_code(out_dtype),
                        flags, 0 if G == H else G)
    y = torch.empty((T, H, P, R), dtype=out_dtype, device="cuda")
    if y_fill is not None:
        y.fill_(y_fill)
    hT = torch.empty((S, H, P, N), dtype=torch.float32, device="cuda")
    ws = m3.workspace(dims, "cuda", varlen=True)
    m3.m3_scan_prefill_varlen(dims, g["cu_seqlens"], g["x"], g["dt"], g["A"], g["lam"],
                              g["theta"], g["B"], g["C"], g["h0"], g["x_prev"], g["B_prev"], y,
                              hT, ws)
    torch.cuda.synchronize()
    return y, hT


def _seq(d, s, a, b, flags):
    """Sequence s (rows a..b) as a batch-1 dense input set."""
    e = {k: d[k][a:b].unsqueeze(0).contiguous() for k in TOK}
    e["A"] = d["A"][a:b].unsqueeze(0).contiguous() if flags & m3.M3_A_PER_TOKEN else d["A"]
    for k in SEQ:
        e[k] = None if d[k] is None else d[k][s:s + 1].contiguous()
    return e


def _run_dense(d, flags=0, out_dtype=torch.float32):
    """One m3_scan_prefill per non-empty sequence; an empty one keeps h0."""
    cu = _cu(d)
    ys, hs = [], []
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        if b == a:
            hs.append(cuda(d["h0"][s:s + 1]) if d["h0"] is not None else
                      torch.zeros((1,) + tuple(d["x"].shape[1:3]) + (d["B"].shape[2],), device="cuda"))
            continue
        e = {k: cuda(v) for k, v in _seq(d, s, a, b, flags).items()}
        y, hT = m3.scan_prefill(e["x"], e["dt"], e["A"], e["lam"], e["theta"], e["B"], e["C"],
                                e["h0"], e["x_prev"], e["B_prev"], flags=flags, out_dtype=out_dtype)
        ys.append(y[0])
        hs.append(hT)
    torch.cuda.synchronize()
    return torch.cat(ys, 0), torch.cat(hs, 0)


def _per_head(t, H, dim):
    return t if t is None or t.shape[dim] == H else t.repeat_interleave(H // t.shape[dim], dim=dim)


def _oracle(d, flags=0):
    """The fp64 oracle on each sequence alone."""
    cu = _cu(d)
    H = d["x"].shape[1]
    ys, hs = [], []
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        if b == a:
            hs.append(cpu64(d["h0"][s:s + 1]) if d["h0"] is not None else
                      np.zeros((1, H, d["x"].shape[2], d["B"].shape[2])))
            continue
        e = _seq(d, s, a, b, flags)
        for k in ("B", "C", "theta"):
            e[k] = _per_head(e[k], H, 2)
        e["B_prev"] = _per_head(e["B_prev"], H, 1)
        r = oracle.scan(*(cpu64(e[k]) for k in ("x", "dt", "A", "lam", "theta", "B", "C", "h0",
                                                 "x_prev", "B_prev")), flags=flags)
        ys.append(r.y[0])
        hs.append(r.hT)
    return np.concatenate(ys, 0), np.concatenate(hs, 0)


def _check(d, flags=0, out_dtype=torch.float32, extra_tol=0.0):
    y, hT = _run_varlen(d, flags, out_dtype)
    yd, hd = _run_dense(d, flags, out_dtype)
    same = torch.equal(y, yd) and torch.equal(hT, hd)
    ry, rh = _oracle(d, flags)
    ey, eh = rel_err(cpu64(y), ry), rel_err(cpu64(hT), rh)
    tol = TOL[d["x"].dtype]
    say(f"  y err {ey:.2e}  hT err {eh:.2e}  (tol {tol:.0e}); equal to per-sequence calls: {same}")
    assert same
    assert ey <= tol + extra_tol and eh <= tol, (ey, eh)


@pytest.mark.parametrize("R", [1, 2, 4])
def test_varlen_mixed_lengths(R):
    w = I.Workload("v", 110, 1, 1, 3, 64, 128, R, 64, "bf16")
    say(f"varlen lengths {LENGTHS} R={R}")
    _check(_packed(w, LENGTHS))


@pytest.mark.parametrize("P,N,R,dt", [
    (16, 16, 1, "f32"), (32, 64, 1, "bf16"), (32, 64, 4, "bf16"), (64, 64, 1, "bf16"),
    (64, 64, 4, "bf16"), (64, 128, 1, "f32"), (64, 128, 4, "f32"),
])
def test_varlen_shapes(P, N, R, dt):
    w = I.Workload("v", 111, 1, 1, 2, P, N, R, 64, dt)
    lengths = [70, 0, 129, 5]
    say(f"varlen P={P} N={N} R={R} {dt} lengths {lengths}")
    _check(_packed(w, lengths))


@pytest.mark.parametrize("R", [1, 4])
def test_varlen_flags_groups_no_prev(R):
    lengths = [100, 64, 1, 90]
    w = I.Workload("v", 112, 1, 1, 4, 64, 128, R, 64, "bf16")
    say(f"varlen groups=2 R={R}")
    _check(_packed(w, lengths, groups=2))
    say(f"varlen no h0, no prev R={R}")
    _check(_packed(w, lengths, prev=False, h0="zero"))
    say(f"varlen theta is angle R={R}")
    _check(_packed(w, lengths), flags=m3.M3_THETA_IS_ANGLE)
    say(f"varlen A per token R={R}")
    d = _packed(w, lengths)
    rng = np.random.default_rng(11)
    d["A"] = torch.from_numpy(-np.exp(rng.uniform(-4, 0, size=(sum(lengths), 4))).astype(np.float32))
    _check(d, flags=m3.M3_A_PER_TOKEN)
    say(f"varlen bf16 y R={R}")
    _check(_packed(w, lengths), out_dtype=torch.bfloat16, extra_tol=2 ** -8)


def test_varlen_offsets_are_clamped():
    """Offsets that fall, leave [0, T] or do not start at 0 are read as the
    library documents: each is clamped into [0, T] and raised to the largest
    offset before it.  Rows outside every sequence keep what y held."""
    w = I.Workload("v", 113, 1, 1, 2, 64, 128, 4, 64, "bf16")
    T = 300
    d = _packed(w, [T])
    raw = [5, 100, 40, 170, 900, 250, -3]          # 6 sequences
    d["cu_seqlens"] = torch.tensor(raw, dtype=torch.int32)
    for k in SEQ:
        d[k] = d[k].repeat((6,) + (1,) * (d[k].dim() - 1)).contiguous()
    y, hT = _run_varlen(d, y_fill=float("nan"))
    eff, run = [], 0
    for v in raw:
        run = max(run, min(max(v, 0), T))
        eff.append(run)
    say(f"  raw offsets {raw} -> {eff}")
    e = dict(d)
    e["cu_seqlens"] = torch.tensor(eff, dtype=torch.int32)
    y2, h2 = _run_varlen(e, y_fill=float("nan"))
    assert torch.equal(hT, h2)
    assert torch.isnan(y[:eff[0]]).all() and torch.isnan(y2[:eff[0]]).all()
    assert torch.equal(y[eff[0]:eff[-1]], y2[eff[0]:eff[-1]])
    assert not torch.isnan(y[eff[0]:eff[-1]]).any()
    # the clamped split against the oracle (rows eff[0]..eff[-1] only)
    sub = dict(e)
    for k in TOK:
        sub[k] = d[k][eff[0]:eff[-1]]
    sub["cu_seqlens"] = torch.tensor([v - eff[0] for v in eff], dtype=torch.int32)
    ry, rh = _oracle(sub)
    assert rel_err(cpu64(y[eff[0]:eff[-1]]), ry) <= TOL[torch.bfloat16]
    assert rel_err(cpu64(hT), rh) <= TOL[torch.bfloat16]


@pytest.mark.parametrize("R", [1, 4])
def test_varlen_hands_off_to_decode(R):
    """Packed prefill, then every sequence decodes 3 more tokens from its
    final state with its last prefill token as the token before: the
    outputs equal the oracle's scan over prompt plus the new tokens."""
    lengths = [77, 1, 150, 64]
    K = 3
    w = I.Workload("v", 114, 1, 1, 3, 64, 128, R, 64, "bf16")
    full = [n + K for n in lengths]
    d = _packed(w, full)                 # prompt rows followed by K decode rows per sequence
    cu = _cu(d)
    pre_rows = np.concatenate([np.arange(cu[s], cu[s] + lengths[s]) for s in range(len(lengths))])
    dec_rows = np.stack([np.arange(cu[s] + lengths[s], cu[s + 1]) for s in range(len(lengths))])
    p = {k: d[k][pre_rows].contiguous() for k in TOK}
    p.update(A=d["A"], h0=d["h0"], x_prev=d["x_prev"], B_prev=d["B_prev"])
    p["cu_seqlens"] = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)
    y_pre, hT = _run_varlen(p)
    last = torch.tensor(np.cumsum(lengths) - 1)
    g = lambda t: cuda(t)
    t = {k: g(d[k][torch.from_numpy(dec_rows)]) for k in TOK}   # [S, K, ...]
    h = hT.clone()
    y_dec = m3.decode_tokens(h, t["x"], t["B"], t["C"], t["dt"], g(d["A"]), t["lam"], t["theta"],
                             x_prev=g(p["x"][last]), B_prev=g(p["B"][last]))
    torch.cuda.synchronize()
    ry, rh = _oracle(d)
    ey_pre = rel_err(cpu64(y_pre), ry[pre_rows])
    ey_dec = rel_err(cpu64(y_dec).reshape((-1,) + ry.shape[1:]), ry[dec_rows.reshape(-1)])
    eh = rel_err(cpu64(h), rh)
    say(f"  prefill y {ey_pre:.2e}  decode y {ey_dec:.2e}  final h {eh:.2e}")
    tol = TOL[torch.bfloat16]
    assert ey_pre <= tol and ey_dec <= tol and eh <= tol


@pytest.mark.parametrize("name", ["siso_prefill_varlen", "mimo_prefill_varlen"])
def test_varlen_serving_mix_full_size(name):
    """The packed serving mix at full size, in the benchmark's launch
    configuration: bit-equal to one call per sequence, and the shortest
    sequences against the oracle in full."""
    w, max_len = I.PACKED[name]
    lengths = I.packed_lengths(w, max_len)
    say(f"{name}: {len(lengths)} sequences, {sum(lengths)} tokens")
    d = I.packed_inputs(w, lengths)
    y, hT = _run_varlen(d)
    yd, hd = _run_dense(d)
    assert torch.equal(y, yd) and torch.equal(hT, hd)
    cu = _cu(d)
    for s in np.argsort(lengths)[:2]:
        a, b = cu[s], cu[s + 1]
        sub = {k: d[k][a:b] for k in TOK}
        sub.update(A=d["A"], h0=None, x_prev=None, B_prev=None,
                   cu_seqlens=torch.tensor([0, b - a], dtype=torch.int32))
        ry, rh = _oracle(sub)
        ey, eh = rel_err(cpu64(y[a:b]), ry), rel_err(cpu64(hT[s:s + 1]), rh)
        say(f"  sequence {s} ({b - a} tokens): y err {ey:.2e}  hT err {eh:.2e}")
        assert ey <= TOL[torch.bfloat16] and eh <= TOL[torch.bfloat16]


@pytest.mark.parametrize("R", [1, 4])
def test_varlen_deterministic_and_nan_stays_in_its_sequence(R):
    """Two calls agree bit for bit.  A NaN in one token of the middle sequence
    stays in that sequence and head: every sequence starts its own chunks, so
    the neighbours packed before and after it never see it, and inside it the
    NaN reaches the outputs from its chunk's first token on (the chunk's masked
    products multiply it by zero)."""
    lengths = [100, 150, 37]
    w = I.Workload("v", 115, 1, 1, 3, 64, 128, R, 64, "bf16")
    d = _packed(w, lengths)
    say(f"varlen determinism and NaN isolation R={R}")
    y1, h1 = _run_varlen(d)
    y2, h2 = _run_varlen(d)
    assert torch.equal(y1.cpu(), y2.cpu()) and torch.equal(h1.cpu(), h2.cpu())
    cu = _cu(d)
    x = d["x"].clone()
    x[cu[1] + 70, 2].view(-1)[5] = float("nan")   # sequence 1, its chunk 1 (tokens 64..127)
    y, hT = _run_varlen(dict(d, x=x))
    bad_y = torch.isnan(y).flatten(2).any(dim=2).cpu()          # [token, head]
    expect = torch.zeros_like(bad_y)
    expect[cu[1] + 64:cu[2], 2] = True
    assert torch.equal(bad_y, expect)
    bad_h = torch.isnan(hT).flatten(2).any(dim=2).cpu()         # [sequence, head]
    assert bad_h[1, 2] and bad_h.sum() == 1
