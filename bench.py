#!/usr/bin/env python3
"""Benchmark of libm3ssm on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Headline: the SISO decode step at B=128, H=64, P=64, N=128 (bf16 inputs, fp32
state carried in HBM): K sequential steps after W warm-up steps, every step a
fresh token from a pool of distinct resident input sets, the state updated in
place.  `value` is the algorithmic HBM traffic of the K steps divided by their
wall time on the GPU (GB/s); `us_per_step` is the same time per step.
`roofline` compares the decode kernel's average duration (HIP events around
each launch, on the launch stream) with the 8 TB/s HBM peak.

In the same run and the same JSON line, under "workloads": the MIMO rank-4
decode step (same shape), the SISO chunked prefill (B=4, T=2048, H=32) and the
MIMO rank-4 long prefill (B=1, T=16384, H=64), each with its own timing and
roofline fraction, and the fp64 CPU oracle timed on a bounded sample of each
workload (`cpu_baseline`, a reported baseline only); also four decode tokens
per call (m3_decode_tokens, the state crossing HBM once per call) at both
decode shapes, the two prefill shapes' tokens packed as sequences of
drawn lengths (m3_scan_prefill_varlen), and the decode steps and prefills
again with the in-kernel B/C preparation (RMS normalisation, weight and
per-head bias of B and C; "_bcprep"), and the gradients of both prefills
(m3_scan_prefill_backward; "siso_prefill_backward", "mimo_prefill_backward").

Prints one JSON line.  Only one GPU is supported: --gpus N > 1 exits.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "decode-step µs & HBM GB/s at B=128,H=64,P=64,N=128; prefill tokens/s"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic bytes (each input read once, outputs written once, state read
# and written once)
def decode_bytes(w, in_bytes=2, out_bytes=4):
    B, H, P, N, R = w.batch, w.nheads, w.headdim, w.dstate, w.rank
    state = 2 * B * H * P * N * 4
    inputs = in_bytes * (2 * B * H * P * R + 3 * B * H * N * R + 2 * B * H + B * H * N // 2)
    return state + inputs + H * 4 + out_bytes * B * H * P * R


def decode_tokens_bytes(w, K, in_bytes=2, out_bytes=4):
    """K tokens in one call: the state once in and once out, every token's
    inputs and outputs once, the token before the first once."""
    B, H, P, N, R = w.batch, w.nheads, w.headdim, w.dstate, w.rank
    state = 2 * B * H * P * N * 4
    per_tok = in_bytes * (B * H * P * R + 2 * B * H * N * R + 2 * B * H + B * H * N // 2)
    prev = in_bytes * (B * H * P * R + B * H * N * R)
    return state + K * per_tok + prev + H * 4 + K * out_bytes * B * H * P * R


def prefill_bytes(w, in_bytes=2, out_bytes=4, h0=False, hT=True, nseq=None):
    """nseq: packed sequences (one final state each) in w's T token rows."""
    B, T, H, P, N, R = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.rank
    inputs = in_bytes * (B * T * H * P * R + 2 * B * T * H * N * R + 2 * B * T * H
                         + B * T * H * N // 2)
    states = (int(h0) + int(hT)) * (nseq or B) * H * P * N * 4
    return inputs + states + H * 4 + out_bytes * B * T * H * P * R


def prefill_flops(w):
    """Dense chunk contractions of the chunked prefill, 2 flops per multiply-add:
    per chunk-head the Gram (QR)^2 N and Y_diag (QR)^2 P over the chunk's QR
    virtual rows, Y_off and the chunk state QR N P each."""
    Q, R, N, P = w.chunk, w.rank, w.dstate, w.headdim
    chunks = w.batch * w.nheads * ((w.seqlen + Q - 1) // Q)
    V = Q * R
    return 2 * chunks * (V * V * (N + P) + 2 * V * N * P)


MFMA_PEAK_TFLOPS = 2500.0   # dense fp16 MFMA (MI355X); the split operands run on it


def source_hash(files):
    """Hash of the named files under the package's csrc/ directory."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_recurrent_sequence_mamba_amd", "csrc")
    for f in sorted(files):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def counters_for(kernel_tag):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (profiles/hbm_counters.json), if it was taken on the current sources of
    that kernel; else None."""
    path = os.path.join(ROOT, "profiles", "hbm_counters.json")
    try:
        with open(path) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        return None
    ent = data.get("kernels", {}).get(kernel_tag)
    if not ent or ent.get("source_hash") != source_hash(ent.get("sources", [])):
        return None
    return ent.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------
def bc_prep_for(w, dev):
    """The in-kernel B/C preparation (weights, per-head biases, eps) of a
    workload's shape, on the device."""
    from linear_recurrent_sequence_mamba_amd import binding as m3
    from linear_recurrent_sequence_mamba_amd import inputs as I
    _, prm = I.bc_prep_inputs(w, {})
    return m3.BCPrep(**{k: prm[k].to(dev) for k in ("B_weight", "C_weight", "B_bias", "C_bias")},
                     eps=prm["eps"])


def bench_decode(name, steps, warmup, pool_n=8, prep=False):
    """prep: with the in-kernel B/C preparation (m3_dims.bc)."""
    import torch
    from linear_recurrent_sequence_mamba_amd import binding as m3
    from linear_recurrent_sequence_mamba_amd import inputs as I

    w = I.WORKLOADS[name]
    dev = torch.device("cuda:0")
    pool_n = max(2, min(pool_n, steps + warmup))
    t0 = time.time()
    pool = []
    for s in range(pool_n):
        d = I.decode_step_inputs(w, s)
        pool.append({k: v.to(dev) for k, v in d.items()})
    log(f"[{name}] generated {pool_n} input sets in {time.time() - t0:.1f}s")
    h = I.decode_state(w).to(dev)
    A = I.head_decay(w).to(dev)
    y = torch.empty((w.batch, w.nheads, w.headdim, w.rank), dtype=torch.float32, device=dev)
    dims = m3.make_dims(w.batch, 1, w.nheads, w.headdim, w.dstate, w.rank, 0, m3.M3_BF16, m3.M3_F32,
                        bc=bc_prep_for(w, dev) if prep else None)
    stream = torch.cuda.current_stream()
    # validate every argument set once through the checked binding ...
    for s in range(pool_n):
        cur, prev = pool[s], pool[(s - 1) % pool_n]
        m3.m3_decode_step(dims, h, cur["x"], prev["x"], cur["B"], prev["B"], cur["C"], cur["dt"],
                          A, cur["lam"], cur["theta"], y)
    torch.cuda.synchronize()
    # ... then launch through the raw entry point (argument marshalling only)
    lib = m3.library()
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    sp = ctypes.c_void_p(stream.cuda_stream)
    args = []
    for s in range(pool_n):
        cur, prev = pool[s], pool[(s - 1) % pool_n]
        args.append((ctypes.byref(dims), p(h), p(cur["x"]), p(prev["x"]), p(cur["B"]), p(prev["B"]),
                     p(cur["C"]), p(cur["dt"]), p(A), p(cur["lam"]), p(cur["theta"]), p(y), sp))

    def launch(s):
        st = lib.m3_decode_step(*args[s % pool_n])
        if st != 0:
            raise RuntimeError(f"m3_decode_step failed: {m3.m3_status_str(st)}")

    for s in range(warmup):
        launch(s)
    torch.cuda.synchronize()

    # stream launches, K steps (reported beside the graph figure)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for s in range(steps):
        launch(warmup + s)
    end.record(stream)
    torch.cuda.synchronize()
    stream_ms = start.elapsed_time(end)

    # the timed K steps: one HIP graph holding the K launches (what a decode
    # loop captures), replayed once untimed to load it, then timed
    g = torch.cuda.CUDAGraph()
    gs = torch.cuda.Stream()
    gs.wait_stream(stream)
    with torch.cuda.stream(gs):
        with torch.cuda.graph(g, stream=gs):
            cap = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            for s in range(steps):
                st = lib.m3_decode_step(*(args[s % pool_n][:-1] + (cap,)))
                if st != 0:
                    raise RuntimeError(m3.m3_status_str(st))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    g.replay()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(end)
    nbytes = decode_bytes(w)
    return dict(workload=w, steps=steps, total_ms=total_ms, step_ms=total_ms / steps,
                stream_step_ms=stream_ms / steps, wall_s=wall, bytes=nbytes, pool=pool_n)


def bench_decode_tokens(name, K, calls, warmup=3, pool_n=4):
    """K decode tokens per call (m3_decode_tokens) at the decode shape: `calls`
    calls captured in one HIP graph, each a fresh set of K tokens."""
    import torch
    from linear_recurrent_sequence_mamba_amd import binding as m3
    from linear_recurrent_sequence_mamba_amd import inputs as I

    w = I.WORKLOADS[name].with_(seqlen=K)
    dev = torch.device("cuda:0")
    pool = []
    for s in range(pool_n):
        d = I.prefill_inputs(w, stream=100 + s)
        pool.append({k: (None if v is None else v.to(dev)) for k, v in d.items() if k != "h0"})
    for s in range(pool_n):   # the token before a set is the last token of the one before it
        prev = pool[(s - 1) % pool_n]
        pool[s]["x_prev"] = prev["x"][:, -1].contiguous()
        pool[s]["B_prev"] = prev["B"][:, -1].contiguous()
    h = I.decode_state(w).to(dev)
    y = torch.empty((w.batch, K, w.nheads, w.headdim, w.rank), dtype=torch.float32, device=dev)
    dims = m3.make_dims(w.batch, K, w.nheads, w.headdim, w.dstate, w.rank, 0, m3.M3_BF16, m3.M3_F32)
    for d in pool:   # validate every argument set through the checked binding
        m3.m3_decode_tokens(dims, h, d["x"], d["x_prev"], d["B"], d["B_prev"], d["C"], d["dt"],
                            d["A"], d["lam"], d["theta"], y)
    torch.cuda.synchronize()
    lib = m3.library()
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    args = [(ctypes.byref(dims), p(h), p(d["x"]), p(d["x_prev"]), p(d["B"]), p(d["B_prev"]),
             p(d["C"]), p(d["dt"]), p(d["A"]), p(d["lam"]), p(d["theta"]), p(y)) for d in pool]
    stream = torch.cuda.current_stream()
    for s in range(warmup):
        lib.m3_decode_tokens(*args[s % pool_n], ctypes.c_void_p(stream.cuda_stream))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    gs = torch.cuda.Stream()
    gs.wait_stream(stream)
    with torch.cuda.stream(gs):
        with torch.cuda.graph(g, stream=gs):
            cap = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            for s in range(calls):
                st = lib.m3_decode_tokens(*args[s % pool_n], cap)
                if st != 0:
                    raise RuntimeError(m3.m3_status_str(st))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    call_ms = e0.elapsed_time(e1) / calls
    nbytes = decode_tokens_bytes(w, K)
    gbs = nbytes / (call_ms * 1e-3) / 1e9
    return dict(tokens_per_call=K, us_per_call=round(call_ms * 1e3, 2),
                us_per_token_step=round(call_ms * 1e3 / K, 2),
                tokens_per_s=round(w.batch * K / (call_ms * 1e-3), 1), algorithmic_bytes=nbytes,
                roofline=dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                              frac=round(gbs / HBM_PEAK_GBS, 4), traffic=counters_for(f"{name}_k{K}"),
                              kernel=f"k_decode_{'siso' if w.rank == 1 else 'mimo'}_tok",
                              timing=f"HIP events around a graph of {calls} calls"))


def bench_prefill(name, steps, warmup, prep=False):
    """prep: with the in-kernel B/C preparation (m3_dims.bc)."""
    import torch
    from linear_recurrent_sequence_mamba_amd import binding as m3
    from linear_recurrent_sequence_mamba_amd import inputs as I

    w = I.WORKLOADS[name]
    dev = torch.device("cuda:0")
    t0 = time.time()
    n_sets = 2 if prefill_bytes(w) < 1e9 else 1   # two sets when one would fit in cache
    sets = []
    for s in range(n_sets):
        d = I.prefill_inputs(w, stream=s)
        sets.append({k: (None if v is None else v.to(dev)) for k, v in d.items()})
    log(f"[{name}] generated {n_sets} input set(s) in {time.time() - t0:.1f}s")
    dims = m3.make_dims(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.rank, w.chunk,
                        m3.M3_BF16, m3.M3_F32, bc=bc_prep_for(w, dev) if prep else None)
    ws = m3.workspace(dims, dev)
    y = torch.empty((w.batch, w.seqlen, w.nheads, w.headdim, w.rank), dtype=torch.float32, device=dev)
    hT = torch.empty((w.batch, w.nheads, w.headdim, w.dstate), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def launch(s):
        d = sets[s % n_sets]
        m3.m3_scan_prefill(dims, d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"], d["C"],
                           None, None, None, y, hT, ws, stream)

    for s in range(warmup):
        launch(s)
    torch.cuda.synchronize()
    ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for s in range(steps):
        ev0[s].record(stream)
        launch(warmup + s)
        ev1[s].record(stream)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in zip(ev0, ev1))
    call_ms = sum(ms) / len(ms)
    return dict(workload=w, steps=steps, call_ms=call_ms, call_p50_ms=ms[len(ms) // 2],
                bytes=prefill_bytes(w), tokens=w.batch * w.seqlen, ws_bytes=ws.numel())


def bench_prefill_varlen(name, steps, warmup):
    """A packed serving mix (m3_scan_prefill_varlen): the same tokens as the
    dense prefill shape, split into sequences of drawn lengths."""
    import torch
    from linear_recurrent_sequence_mamba_amd import binding as m3
    from linear_recurrent_sequence_mamba_amd import inputs as I

    w, max_len = I.PACKED[name]
    lengths = I.packed_lengths(w, max_len)
    dev = torch.device("cuda:0")
    t0 = time.time()
    d = {k: (None if v is None else v.to(dev)) for k, v in I.packed_inputs(w, lengths).items()}
    log(f"[{name}] {len(lengths)} sequences, generated in {time.time() - t0:.1f}s")
    S, T = len(lengths), w.seqlen
    dims = m3.make_dims(S, T, w.nheads, w.headdim, w.dstate, w.rank, w.chunk, m3.M3_BF16, m3.M3_F32)
    ws = m3.workspace(dims, dev, varlen=True)
    y = torch.empty((T, w.nheads, w.headdim, w.rank), dtype=torch.float32, device=dev)
    hT = torch.empty((S, w.nheads, w.headdim, w.dstate), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def launch():
        m3.m3_scan_prefill_varlen(dims, d["cu_seqlens"], d["x"], d["dt"], d["A"], d["lam"],
                                  d["theta"], d["B"], d["C"], None, None, None, y, hT, ws, stream)

    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for s in range(steps):
        ev0[s].record(stream)
        launch()
        ev1[s].record(stream)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in zip(ev0, ev1))
    call_ms = sum(ms) / len(ms)
    return dict(workload=w, steps=steps, call_ms=call_ms, call_p50_ms=ms[len(ms) // 2],
                bytes=prefill_bytes(w, nseq=S), tokens=T, ws_bytes=ws.numel(), nseq=S,
                lengths=dict(min=min(lengths), max=max(lengths), mean=round(T / S, 1)))


def backward_bytes(w, in_bytes=2, dy_bytes=4):
    """Inputs and dy read once, every gradient written once (fp32)."""
    B, T, H, P, N, R = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.rank
    tok = B * T * H
    inputs = in_bytes * tok * (P * R + 2 * N * R + 2 + N // 2) + dy_bytes * tok * P * R
    grads = 4 * tok * (P * R + 2 * N * R + 2 + N // 2) + 4 * H
    return inputs + grads


def bench_backward(name, steps, warmup):
    """m3_scan_prefill_backward at a prefill workload's shape (fp32 dy)."""
    import torch
    from linear_recurrent_sequence_mamba_amd import binding as m3
    from linear_recurrent_sequence_mamba_amd import inputs as I

    w = I.WORKLOADS[name]
    dev = torch.device("cuda:0")
    d = {k: (None if v is None else v.to(dev)) for k, v in I.prefill_inputs(w).items()}
    gen = torch.Generator(device="cpu").manual_seed(w.cfg_id)
    dy = torch.randn(tuple(d["x"].shape), generator=gen).to(dev)
    dims = m3.make_dims(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.rank, w.chunk,
                        m3.M3_BF16, m3.M3_F32)
    n = m3.m3_prefill_backward_workspace_size(dims)
    ws = torch.empty((n + 15) // 16 * 16, dtype=torch.uint8, device=dev)
    f32 = torch.float32
    grads = {k: torch.empty(d[k].shape, dtype=f32, device=dev)
             for k in ("x", "dt", "A", "lam", "theta", "B", "C")}
    stream = torch.cuda.current_stream()

    def launch():
        m3.m3_scan_prefill_backward(dims, d["x"], d["dt"], d["A"], d["lam"], d["theta"], d["B"],
                                    d["C"], None, None, None, dy, None, grads, ws, stream)

    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for e0, e1 in ev:
        e0.record(stream)
        launch()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    call_ms = sum(ms) / len(ms)
    nbytes = backward_bytes(w)
    return dict(ms_per_call=round(call_ms, 4), p50_ms=round(ms[len(ms) // 2], 4),
                tokens_per_s=round(w.batch * w.seqlen / (call_ms * 1e-3), 1),
                algorithmic_bytes=nbytes,
                hbm_frac=round(nbytes / (call_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                note="forward chunk states recomputed inside the call; fp32 dy and gradients")


def copy_reference(state_bytes, reps=50):
    """A plain device copy of a state-sized buffer (torch's copy kernel): read
    + write of the same byte count the decode step streams.  Context for the
    8 TB/s nominal peak; not a kernel of this library."""
    import torch
    n = state_bytes // 4
    src = torch.empty(n, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    out = dict(bytes=2 * state_bytes, us=round(ms * 1e3, 2), gbs=round(2 * state_bytes / (ms * 1e-3) / 1e9, 1),
               kernel="torch copy_ (read + write of a 268 MB fp32 buffer)")
    # in-place updates (read and write the same buffer, as the decode state
    # is): at the state's size, which the 256 MB last-level cache partly
    # holds between passes, and at twice that, which it cannot
    for mult in (1, 2):
        buf = torch.ones(n * mult, dtype=torch.float32, device="cuda:0")
        for _ in range(3):
            buf.mul_(1.0)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            buf.mul_(1.0)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        nb = 2 * state_bytes * mult
        out[f"inplace_x{mult}"] = dict(bytes=nb, us=round(ms * 1e3, 2), gbs=round(nb / (ms * 1e-3) / 1e9, 1),
                                       kernel=f"torch mul_ in place on a {state_bytes * mult // 2**20} MiB fp32 buffer")
        del buf
    return out


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle as it stands, on a bounded sample
def cpu_decode(name, budget_s=8.0):
    from linear_recurrent_sequence_mamba_amd import inputs as I
    from oracle import oracle
    import numpy as np

    w = I.WORKLOADS[name]
    nb = 16  # batch rows of the sample; every head
    d = I.decode_step_inputs(w, 0)
    f = {k: I.to_f64(v)[:nb] for k, v in d.items()}
    h = I.to_f64(I.decode_state(w))[:nb]
    A = I.to_f64(I.head_decay(w))
    oracle.load()
    steps, t0 = 0, time.perf_counter()
    while True:
        y, h = oracle.decode_step(h, f["x"], f["x"], f["B"], f["B"], f["C"], f["dt"], A,
                                  f["lam"], f["theta"])
        steps += 1
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    full_s = el / steps * (w.batch / nb)
    return dict(value=round(decode_bytes(w) / full_s / 1e9, 3), unit="GB/s",
                us_per_step=round(full_s * 1e6, 1), cores=oracle.max_threads(), kind="oracle",
                sample=f"{steps} decode steps of {nb} of {w.batch} batch rows x {w.nheads} heads "
                       f"(fp64, OpenMP over (b,h)); time scaled by {w.batch // nb} to the full step")


def cpu_prefill(name, heads, tokens, budget_note=""):
    from linear_recurrent_sequence_mamba_amd import inputs as I
    from oracle import oracle

    w = I.WORKLOADS[name]
    ws = w.with_(batch=1, seqlen=tokens, nheads=heads)
    d = I.prefill_inputs(ws)
    f = {k: I.to_f64(v) for k, v in d.items()}
    t0 = time.perf_counter()
    oracle.scan(f["x"], f["dt"], f["A"], f["lam"], f["theta"], f["B"], f["C"])
    el = time.perf_counter() - t0
    # heads and tokens are independent/sequential units of identical work
    full_s = el * (w.nheads / heads) * (w.batch) * (w.seqlen / tokens)
    return dict(value=round(w.batch * w.seqlen / full_s, 1), unit="tokens/s",
                cores=oracle.max_threads(), kind="oracle",
                sample=f"{heads} heads x {tokens} tokens of one sequence (fp64); time scaled "
                       f"linearly to {w.batch} x {w.seqlen} tokens x {w.nheads} heads")


# ---------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default="", help="comma list of workloads to run (default all)")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decode and prefill kernels run on a "
              "single MI355X; multi-GPU runs are not part of this library.", file=sys.stderr)
        sys.exit(2)
    if a.steps < 1 or a.warmup < 0:
        ap.error("--steps must be >= 1 and --warmup >= 0")

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    from linear_recurrent_sequence_mamba_amd import binding as m3
    m3.library()  # fail loudly if the HIP library is missing
    only = set(x for x in a.only.split(",") if x)
    want = lambda n: not only or n in only

    res = {}
    if want("siso_decode"):
        res["siso_decode"] = bench_decode("siso_decode", a.steps, a.warmup)
    if want("mimo_decode"):
        res["mimo_decode"] = bench_decode("mimo_decode", a.steps, a.warmup)
    if want("siso_prefill"):
        res["siso_prefill"] = bench_prefill("siso_prefill", a.prefill_steps, 2)
    if want("mimo_prefill"):
        res["mimo_prefill"] = bench_prefill("mimo_prefill", a.prefill_steps, 2)
    for name in ("siso_prefill_varlen", "mimo_prefill_varlen"):
        if want(name):
            res[name] = bench_prefill_varlen(name, a.prefill_steps, 2)
    prep = {}   # the same shapes with the in-kernel B/C preparation
    for name in ("siso_decode", "mimo_decode"):
        if want(name + "_bcprep"):
            prep[name] = bench_decode(name, a.steps, a.warmup, prep=True)
    for name in ("siso_prefill", "mimo_prefill"):
        if want(name + "_bcprep"):
            prep[name] = bench_prefill(name, a.prefill_steps, 2, prep=True)
    bwd = {}
    if want("siso_prefill_backward"):
        bwd["siso_prefill_backward"] = bench_backward("siso_prefill", a.prefill_steps, 2)
    if want("mimo_prefill_backward"):
        bwd["mimo_prefill_backward"] = bench_backward("mimo_prefill", a.prefill_steps, 2)
    tok = {}
    for base in ("siso_decode", "mimo_decode"):
        if want(base + "_k4"):
            tok[base + "_k4"] = bench_decode_tokens(base, 4, 100)

    copy_ref = None
    if "siso_decode" in res:
        from linear_recurrent_sequence_mamba_amd import inputs as I
        w = I.WORKLOADS["siso_decode"]
        copy_ref = copy_reference(w.batch * w.nheads * w.headdim * w.dstate * 4)

    cpu = {}
    if not a.no_cpu_baseline:
        t0 = time.time()
        if "siso_decode" in res:
            cpu["siso_decode"] = cpu_decode("siso_decode", 8.0)
        if "mimo_decode" in res:
            cpu["mimo_decode"] = cpu_decode("mimo_decode", 6.0)
        if "siso_prefill" in res:
            cpu["siso_prefill"] = cpu_prefill("siso_prefill", heads=8, tokens=2048)
        if "mimo_prefill" in res:
            cpu["mimo_prefill"] = cpu_prefill("mimo_prefill", heads=4, tokens=4096)
        log(f"cpu baselines took {time.time() - t0:.1f}s")

    def decode_entry(r, tag):
        w = r["workload"]
        gbs = r["bytes"] / (r["step_ms"] * 1e-3) / 1e9
        traffic = counters_for(tag)
        return dict(
            us_per_step=round(r["step_ms"] * 1e3, 2),
            stream_launch_us_per_step=round(r["stream_step_ms"] * 1e3, 2),
            hbm_gbs=round(gbs, 1), tokens_per_s=round(w.batch / (r["step_ms"] * 1e-3), 1),
            algorithmic_bytes=r["bytes"], input_pool=r["pool"],
            roofline=dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                          frac=round(gbs / HBM_PEAK_GBS, 4), traffic=traffic,
                          kernel=f"k_decode_{'siso' if w.rank == 1 else 'mimo'}",
                          timing="HIP events around a graph of the K launches (one kernel per step)"),
            cpu_baseline=cpu.get(tag))

    def prefill_entry(r, tag):
        ach = r["bytes"] / (r["call_ms"] * 1e-3) / 1e9
        if "nseq" in r:   # packed sequences: no separate counters or CPU leg
            return dict(
                ms_per_call=round(r["call_ms"], 4), p50_ms=round(r["call_p50_ms"], 4),
                tokens_per_s=round(r["tokens"] / (r["call_ms"] * 1e-3), 1),
                sequences=r["nseq"], lengths=r["lengths"], algorithmic_bytes=r["bytes"],
                workspace_bytes=r["ws_bytes"], hbm_frac=round(ach / HBM_PEAK_GBS, 4))
        fl = prefill_flops(r["workload"])
        tf = fl / (r["call_ms"] * 1e-3) / 1e12
        return dict(
            ms_per_call=round(r["call_ms"], 4), p50_ms=round(r["call_p50_ms"], 4),
            tokens_per_s=round(r["tokens"] / (r["call_ms"] * 1e-3), 1),
            algorithmic_bytes=r["bytes"], workspace_bytes=r["ws_bytes"],
            roofline=dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                          frac=round(ach / HBM_PEAK_GBS, 4), traffic=counters_for(tag),
                          kernel="whole call (k_chunk_state + k_state_pass + k_chunk_output)"),
            mfma=dict(flops=fl, achieved=round(tf, 1), peak=MFMA_PEAK_TFLOPS, unit="TFLOP/s",
                      frac=round(tf / MFMA_PEAK_TFLOPS, 4),
                      counting="dense chunk contractions: Gram (QR)^2 N, Y_diag (QR)^2 P, Y_off and "
                               "chunk state QR N P each, 2 flops per multiply-add"),
            cpu_baseline=cpu.get(tag))

    workloads = {}
    for tag, r in res.items():
        workloads[tag] = decode_entry(r, tag) if "decode" in tag else prefill_entry(r, tag)
    workloads.update(tok)   # several tokens per call (m3_decode_tokens), same shapes
    for k, e in bwd.items():
        base = k.replace("_backward", "")
        if base in workloads:
            e["call_time_vs_forward"] = round(e["ms_per_call"] / workloads[base]["ms_per_call"], 3)
        workloads[k] = e
    for base, r in prep.items():
        if "decode" in base:
            e = dict(us_per_step=round(r["step_ms"] * 1e3, 2),
                     tokens_per_s=round(r["workload"].batch / (r["step_ms"] * 1e-3), 1),
                     hbm_frac=round(r["bytes"] / (r["step_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))
            if base in workloads:
                e["step_time_vs_plain"] = round(e["us_per_step"] / workloads[base]["us_per_step"], 3)
        else:
            e = dict(ms_per_call=round(r["call_ms"], 4),
                     tokens_per_s=round(r["tokens"] / (r["call_ms"] * 1e-3), 1))
            if base in workloads:
                e["call_time_vs_plain"] = round(e["ms_per_call"] / workloads[base]["ms_per_call"], 3)
        workloads[base + "_bcprep"] = e
    for base in ("siso_prefill", "mimo_prefill"):
        if base in workloads and base + "_varlen" in workloads:
            workloads[base + "_varlen"]["tokens_per_s_vs_dense"] = round(
                workloads[base + "_varlen"]["tokens_per_s"] / workloads[base]["tokens_per_s"], 3)

    head = res.get("siso_decode")
    line = {"metric": METRIC}
    if head is not None:
        e = workloads["siso_decode"]
        line.update(value=e["hbm_gbs"], unit="GB/s", n_gpus=1, steps=a.steps, warmup=a.warmup,
                    ms_per_step=round(head["step_ms"], 5), us_per_step=e["us_per_step"],
                    higher_is_better=True, scaling="weak", vs_baseline=None, dtype="f32",
                    data="synthetic",
                    config={"workload": "SISO decode step B=128 H=64 P=64 N=128, bf16 inputs, "
                                        "fp32 state in HBM updated in place",
                            "batch": 128, "nheads": 64, "headdim": 64, "dstate": 128, "rank": 1,
                            "input_dtype": "bf16", "state_dtype": "f32", "parallelism": "none"},
                    roofline=e["roofline"], cpu_baseline=e["cpu_baseline"])
    if "mimo_decode" in workloads and "siso_decode" in workloads:
        workloads["mimo_decode"]["step_time_vs_siso"] = round(
            workloads["mimo_decode"]["us_per_step"] / workloads["siso_decode"]["us_per_step"], 3)
    line["workloads"] = workloads
    if copy_ref is not None:
        line["hbm_copy_reference"] = copy_ref
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
