#!/usr/bin/env python3
"""Benchmark of libm3ssm on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Headline: the SISO decode step at B=128, H=64, P=64, N=128 (bf16 inputs, fp32
state carried in HBM): K sequential steps after W warm-up steps, every step a
fresh token from a pool of distinct resident input sets, the state updated in
place.  The K launches are captured in one HIP graph, replayed 11 times with HIP
events around each replay on the launch stream; `value` is the algorithmic HBM
traffic of the K steps divided by the median replay's time (GB/s) and
`us_per_step` the same time per step (with the replays' spread).  `roofline`
compares that rate with the 8 TB/s HBM peak; `traffic` is the counter-measured
HBM bytes per launch when the committed counter summary matches the sources.
The same steps alternating between two states larger together than the
last-level cache are reported as "*_decode_cold".

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


def _replay_ms(g, stream, replays):
    """Per-replay times (ms) of a captured graph, HIP events on `stream`."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(replays)]
    for e0, e1 in ev:
        e0.record(stream)
        g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in ev]


def _spread(ms, per):
    """Median and range of per-replay times, divided by `per` (µs)."""
    v = sorted(m / per * 1e3 for m in ms)
    return dict(median=round(v[len(v) // 2], 2), min=round(v[0], 2), max=round(v[-1], 2),
                replays=len(v))


def bench_decode(name, steps, warmup, pool_n=8, prep=False, replays=11, cold=False):
    """prep: with the in-kernel B/C preparation (m3_dims.bc).  cold: step s
    updates state s % 2 of two separate states, so that every step streams a
    state the other one has pushed out of the 256 MB last-level cache."""
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
    nstate = 2 if cold else 1
    hs = [I.decode_state(w).to(dev) for _ in range(nstate)]
    A = I.head_decay(w).to(dev)
    y = torch.empty((w.batch, w.nheads, w.headdim, w.rank), dtype=torch.float32, device=dev)
    dims = m3.make_dims(w.batch, 1, w.nheads, w.headdim, w.dstate, w.rank, 0, m3.M3_BF16, m3.M3_F32,
                        bc=bc_prep_for(w, dev) if prep else None)
    stream = torch.cuda.current_stream()
    # validate every argument set once through the checked binding ...
    for s in range(pool_n):
        cur, prev = pool[s], pool[(s - 1) % pool_n]
        for h in hs:
            m3.m3_decode_step(dims, h, cur["x"], prev["x"], cur["B"], prev["B"], cur["C"],
                              cur["dt"], A, cur["lam"], cur["theta"], y)
    torch.cuda.synchronize()
    # ... then launch through the raw entry point (argument marshalling only)
    lib = m3.library()
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    sp = ctypes.c_void_p(stream.cuda_stream)

    def args(s, strm):
        cur, prev = pool[s % pool_n], pool[(s - 1) % pool_n]
        return (ctypes.byref(dims), p(hs[s % nstate]), p(cur["x"]), p(prev["x"]), p(cur["B"]),
                p(prev["B"]), p(cur["C"]), p(cur["dt"]), p(A), p(cur["lam"]), p(cur["theta"]),
                p(y), strm)

    def launch(s):
        st = lib.m3_decode_step(*args(s, sp))
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
    # loop captures), replayed once untimed to load it, then `replays` times,
    # each replay timed on its own; the median replay is the figure
    g = torch.cuda.CUDAGraph()
    gs = torch.cuda.Stream()
    gs.wait_stream(stream)
    with torch.cuda.stream(gs):
        with torch.cuda.graph(g, stream=gs):
            cap = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            for s in range(steps):
                st = lib.m3_decode_step(*args(s, cap))
                if st != 0:
                    raise RuntimeError(m3.m3_status_str(st))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ms = _replay_ms(g, stream, replays)
    wall = time.perf_counter() - wall0
    total_ms = sorted(ms)[len(ms) // 2]
    nbytes = decode_bytes(w)
    return dict(workload=w, steps=steps, total_ms=total_ms, step_ms=total_ms / steps,
                stream_step_ms=stream_ms / steps, wall_s=wall, bytes=nbytes, pool=pool_n,
                spread=_spread(ms, steps), states=nstate)


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
                              kernel="k_decode_siso_tok" if w.rank == 1 else "k_decode_mimo_grp",
                              timing=f"HIP events around a graph of {calls} calls"))


def default_chunk(rank):
    """The chunk length a prefill with m3_dims.chunk = 0 takes (see m3ssm.h)."""
    return 128 if rank == 1 else 64


def bench_prefill(name, steps, warmup, prep=False, chunk=0):
    """prep: with the in-kernel B/C preparation (m3_dims.bc).  chunk: the
    chunk length to ask for (0: the library's default for the shape; the
    result does not depend on it)."""
    import torch
    from linear_recurrent_sequence_mamba_amd import binding as m3
    from linear_recurrent_sequence_mamba_amd import inputs as I

    w = I.WORKLOADS[name].with_(chunk=chunk)
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
                bytes=prefill_bytes(w), tokens=w.batch * w.seqlen, ws_bytes=ws.numel(),
                chunk=chunk or default_chunk(w.rank))


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
    dims = m3.make_dims(S, T, w.nheads, w.headdim, w.dstate, w.rank, 0, m3.M3_BF16, m3.M3_F32)
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
    dims = m3.make_dims(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.rank, 64,
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
def cpu_decode(name, budget_s=8.0, nthreads=0, nb=16):
    """nthreads 0: every host thread (OpenMP over (b, h)); nb batch rows of
    the sample, every head."""
    from linear_recurrent_sequence_mamba_amd import inputs as I
    from oracle import oracle

    w = I.WORKLOADS[name]
    d = I.decode_step_inputs(w, 0)
    f = {k: I.to_f64(v)[:nb] for k, v in d.items()}
    h = I.to_f64(I.decode_state(w))[:nb]
    A = I.to_f64(I.head_decay(w))
    oracle.load()
    steps, t0 = 0, time.perf_counter()
    while True:
        y, h = oracle.decode_step(h, f["x"], f["x"], f["B"], f["B"], f["C"], f["dt"], A,
                                  f["lam"], f["theta"], nthreads=nthreads)
        steps += 1
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    full_s = el / steps * (w.batch / nb)
    cores = nthreads or oracle.max_threads()
    return dict(value=round(decode_bytes(w) / full_s / 1e9, 3), unit="GB/s",
                us_per_step=round(full_s * 1e6, 1), cores=cores, kind="oracle",
                sample=f"{steps} decode steps of {nb} of {w.batch} batch rows x {w.nheads} heads "
                       f"(fp64, {cores} thread{'s' if cores > 1 else ''}, OpenMP over (b,h)); "
                       f"mean time scaled by {w.batch // nb} to the full step")


def cpu_prefill(name, heads, tokens, nthreads=0):
    from linear_recurrent_sequence_mamba_amd import inputs as I
    from oracle import oracle

    w = I.WORKLOADS[name]
    ws = w.with_(batch=1, seqlen=tokens, nheads=heads)
    d = I.prefill_inputs(ws)
    f = {k: I.to_f64(v) for k, v in d.items()}
    t0 = time.perf_counter()
    oracle.scan(f["x"], f["dt"], f["A"], f["lam"], f["theta"], f["B"], f["C"], nthreads=nthreads)
    el = time.perf_counter() - t0
    # heads and tokens are independent/sequential units of identical work
    full_s = el * (w.nheads / heads) * (w.batch) * (w.seqlen / tokens)
    cores = nthreads or oracle.max_threads()
    return dict(value=round(w.batch * w.seqlen / full_s, 1), unit="tokens/s",
                cores=cores, kind="oracle",
                sample=f"{heads} heads x {tokens} tokens of one sequence (fp64, {cores} "
                       f"thread{'s' if cores > 1 else ''}); time scaled linearly to "
                       f"{w.batch} x {w.seqlen} tokens x {w.nheads} heads")


def with_single_thread(all_cores, one):
    """The all-core baseline with the one-thread run beside it."""
    all_cores = dict(all_cores)
    all_cores["single_thread"] = {k: one[k] for k in ("value", "unit", "cores", "sample")}
    return all_cores


# ---------------------------------------------------------------------------
# The rocprofv3 summaries under profiles/, written from the CSV files of
# profiled runs of this script (no GPU needed):
#   python bench.py --summarize-profiles STATS_DIR FETCH_DIR WRITE_DIR BENCH_JSON
#   python bench.py --summarize-sq SQ1_DIR SQ2_DIR
#   python bench.py --summarize-sq-decode SQ1_DIR SQ2_DIR
PROFILE_COPY_BYTES = 268435456   # the device copy of copy_reference(), the counters' calibration
SRC_DECODE = ["decode.hip", "m3_device.h", "m3_launch.h"]
SRC_TOKENS = ["decode_tokens.hip", "m3_device.h", "m3_launch.h"]
SRC_PREFILL = ["prefill.hip", "mfma_pol.h", "chunk_common.h", "m3_device.h", "m3_launch.h"]
SRC_BACKWARD = ["backward.hip", "backward_mma.hip"] + SRC_PREFILL
PROF_STATS_CMD = ("rocprofv3 --kernel-trace --stats -f csv -d gpurun_out/prof_default -o bench -- "
                  "python3 bench.py --steps 200 > gpurun_out/prof_bench.json")
PROF_PMC_CMD = ("rocprofv3 --pmc {c} -f csv -d gpurun_out/pmc_{d} -o bench -- "
                "python3 bench.py --steps 100 --no-cpu-baseline")
PROF_SUM_CMD = ("python3 bench.py --summarize-profiles gpurun_out/prof_default gpurun_out/pmc_fetch "
                "gpurun_out/pmc_write gpurun_out/prof_bench.json")
SQ_ARGS = ("--only siso_prefill,mimo_prefill,siso_prefill_backward,mimo_prefill_backward "
           "--no-cpu-baseline --prefill-steps 2")
SQ_ARGS_DECODE = "--only mimo_decode,mimo_decode_k4 --no-cpu-baseline --steps 20 --warmup 2"
SQ_SETS = ("SQ_WAVES SQ_BUSY_CU_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_INSTS_VALU "
           "SQ_INSTS_LDS SQ_WAVE_CYCLES SQ_BUSY_CYCLES",
           "SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_LDS_BANK_CONFLICT SQ_WAIT_INST_ANY "
           "SQ_ACTIVE_INST_ANY SQ_INSTS_SALU")
MFMA_BF16_FLOPS = 2 * 16 * 16 * 32   # one v_mfma_f32_16x16x32_bf16
MFMA_F32_FLOPS = 2 * 16 * 16 * 4     # one v_mfma_f32_16x16x4_f32 (the decode kernels' only MFMA)
MFMA_F32_PEAK_TFLOPS = 157.3         # dense fp32 matrix (MI355X)
PREFILL_KERNELS = ("k_chunk_state", "k_state_pass", "k_chunk_output", "k_varlen_", "k_bwd_")


def _prof_short(name):
    """A kernel's template name without namespaces, return type and arguments."""
    n = name.replace("(anonymous namespace)::", "").replace("m3::", "")
    if n.endswith(")"):   # drop the argument list
        depth = 0
        for i in range(len(n) - 1, -1, -1):
            depth += {")": 1, "(": -1}.get(n[i], 0)
            if depth == 0:
                n = n[:i]
                break
    return n.replace("void ", "").strip()


def _prof_csv(d, suffix):
    import csv
    for root, _, files in sorted(os.walk(d)):
        for f in sorted(files):
            if f.endswith(suffix):
                with open(os.path.join(root, f), newline="") as fh:
                    return list(csv.DictReader(fh))
    raise SystemExit(f"no *{suffix} under {d}")


def _prof_grid(r):
    if r.get("Grid_Size"):
        return int(r["Grid_Size"])
    return int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])


def _prof_calls(disp):
    """(short name, grid, value) in dispatch order -> the prefill calls: a call
    is a run of prefill kernels that ends at any other kernel or where its
    first kernel (name and grid) comes again."""
    calls, cur = [], None
    for s, g, v in disp:
        if not s.startswith(PREFILL_KERNELS):
            if cur:
                calls.append(cur)
            cur = None
            continue
        if cur and (s, g) == cur[0][:2]:
            calls.append(cur)
            cur = None
        if cur is None:
            cur = []
        cur.append((s, g, v))
    if cur:
        calls.append(cur)
    return calls


def _prof_flavour(sig):
    """The bench workload a call's kernel sequence belongs to."""
    import re
    names = [s for s, _ in sig]
    rank = 1
    for n in names:
        m = re.match(r"k_chunk_state<[^>]*, (\d+), (?:true|false)", n) or re.match(r"k_bwd_u<[^>]*, (\d+)>", n)
        if m:
            rank = int(m.group(1))
    base = "mimo_prefill" if rank > 1 else "siso_prefill"
    if any(n.startswith("k_bwd_") for n in names):
        return base + "_backward"
    if any(n.startswith("k_varlen") for n in names):
        return base + "_varlen"
    if any(n.startswith(("k_chunk_state", "k_chunk_output")) and ", true" in n for n in names):
        return base + "_bcprep"
    return base


def _prof_call_means(disp):
    """flavour -> (kernel signature, mean value per kernel position, calls)."""
    calls = _prof_calls(disp)
    sigs, per = [], {}
    for c in calls:
        sig = tuple((s, g) for s, g, _ in c)
        if sig not in sigs:
            sigs.append(sig)
        per.setdefault(sigs.index(sig), []).append([v for _, _, v in c])
    out = {}
    for i, vals in per.items():
        cols = list(zip(*vals))
        out[_prof_flavour(sigs[i])] = (sigs[i], [sum(c) / len(c) for c in cols], len(vals))
    return out


def _prof_counter(d, counter):
    rs = [r for r in _prof_csv(d, "counter_collection.csv") if r.get("Counter_Name", counter) == counter]
    rs.sort(key=lambda r: int(r["Dispatch_Id"]))
    return [(_prof_short(r["Kernel_Name"]), _prof_grid(r), float(r["Counter_Value"]), r["Kernel_Name"])
            for r in rs]


def summarize_profiles(stats_dir, fetch_dir, write_dir, bench_json, out_dir):
    """kernel_stats_default_bench.txt, hbm_counters_default_bench.txt and
    hbm_counters.json from a --kernel-trace --stats run and a FETCH_SIZE and a
    WRITE_SIZE run of the default bench."""
    import re
    fetch, write = _prof_counter(fetch_dir, "FETCH_SIZE"), _prof_counter(write_dir, "WRITE_SIZE")
    with open(bench_json) as fh:
        W = json.loads(fh.read().strip().splitlines()[-1])["workloads"]

    def means(disp):
        acc, full = {}, {}
        for s, g, v, n in disp:
            acc.setdefault((s, g), []).append(v)
            full[(s, g)] = n
        return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}, full

    fm, fullname = means(fetch)
    wm, _ = means(write)
    # calibration: the device copy of PROFILE_COPY_BYTES (its WRITE_SIZE nearest that size)
    cw = min(((v, s, g) for s, g, v, _ in write if "copy" in s.lower()),
             key=lambda t: abs(t[0] - PROFILE_COPY_BYTES / 1024))
    cfv = [v for s, g, v, _ in fetch if (s, g) == (cw[1], cw[2])]
    cf = sum(cfv) / len(cfv)
    fs, wsc = PROFILE_COPY_BYTES / 1024 / cf, PROFILE_COPY_BYTES / 1024 / cw[0]

    def hbm(key):
        f, n = fm[key]
        w = wm.get(key, (0.0, 0))[0]
        return f * 1024 * fs + w * 1024 * wsc, f, w, n

    fcm = _prof_call_means([(s, g, v) for s, g, v, _ in fetch])
    wcm = _prof_call_means([(s, g, v) for s, g, v, _ in write])
    call_bytes = {}
    for kind, (sig, fv, ncalls) in fcm.items():
        wsig, wv, _ = wcm[kind]
        assert wsig == sig, kind
        per_k = [(sig[i][0], fv[i], wv[i], fv[i] * 1024 * fs + wv[i] * 1024 * wsc) for i in range(len(sig))]
        call_bytes[kind] = (sum(x[3] for x in per_k), sig, per_k, ncalls)

    def is_m3(n):
        return "m3::" in n

    def bools(s):
        return re.findall(r"\b(true|false)\b", s)

    def match(prefix, pred=lambda s: True):
        ks = [k for k in fm if k[0].startswith(prefix) and pred(k[0])]
        return max(ks, key=lambda k: fm[k][1]) if ks else None   # several grids: the most dispatched

    out = {"note": "rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE (KiB per dispatch), mean over dispatches of one "
                   "kernel and grid, scaled by the factors a 268435456-byte device copy reads in the same run",
           "fetch_scale": round(fs, 4), "write_scale": round(wsc, 4), "kernels": {}}
    K = out["kernels"]
    for key in sorted(fm):
        if not is_m3(fullname[key]):
            continue
        b, f, w, n = hbm(key)
        s = key[0]
        src = (SRC_TOKENS if "_tok<" in s or "_grp<" in s else SRC_DECODE if s.startswith("k_decode")
               else SRC_BACKWARD if s.startswith("k_bwd") else SRC_PREFILL)
        K[f"{fullname[key]} grid {key[1]}"] = dict(
            kernel=fullname[key], grid=key[1], fetch_kib=round(f, 1), write_kib=round(w, 1), dispatches=n,
            hbm_bytes_per_launch=round(b), sources=src, source_hash=source_hash(src))
    last3 = lambda v: lambda s: bools(s)[-3:] == v
    tags = {
        "siso_decode": match("k_decode_siso<", last3(["true", "false", "false"])),
        "mimo_decode": match("k_decode_mimo<", last3(["true", "false", "false"])),
        "siso_decode_bcprep": match("k_decode_siso<", last3(["true", "true", "false"])),
        "mimo_decode_bcprep": match("k_decode_mimo<", last3(["true", "true", "false"])),
        "siso_decode_k4": match("k_decode_siso_tok<"),
        "mimo_decode_k4": match("k_decode_mimo_grp<"),
    }
    for tag, key in tags.items():
        if key is None:
            continue
        b, f, w, n = hbm(key)
        base = tag.replace("_bcprep", "")
        alg = (W.get(tag) or {}).get("algorithmic_bytes") or (W.get(base) or {}).get("algorithmic_bytes")
        src = SRC_TOKENS if "k4" in tag else SRC_DECODE
        K[tag] = dict(kernel=fullname[key], fetch_kib=round(f, 1), write_kib=round(w, 1), dispatches=n,
                      hbm_bytes_per_launch=round(b), sources=src, source_hash=source_hash(src),
                      algorithmic_bytes=alg, traffic_over_algorithmic=round(b / alg, 4) if alg else None)
    for kind, (tot, sig, per_k, ncalls) in call_bytes.items():
        base = kind.replace("_bcprep", "")
        alg = (W.get(kind) or {}).get("algorithmic_bytes") or (W.get(base) or {}).get("algorithmic_bytes")
        src = SRC_BACKWARD if "backward" in kind else SRC_PREFILL
        K[kind] = dict(kernel="whole call: " + ", ".join(s for s, g in sig), hbm_bytes_per_launch=round(tot),
                       algorithmic_bytes=alg, traffic_over_algorithmic=round(tot / alg, 4) if alg else None,
                       sources=src, source_hash=source_hash(src), calls=ncalls,
                       per_kernel=[dict(kernel=k_, fetch_kib=round(f_, 1), write_kib=round(w_, 1),
                                        hbm_mb=round(b_ / 1e6, 1)) for k_, f_, w_, b_ in per_k])
    with open(os.path.join(out_dir, "hbm_counters.json"), "w") as fh:
        json.dump(out, fh, indent=1)

    # kernel statistics and the prefill calls' kernel times (from the trace)
    lines = sorted(((float(r["Percentage"]), _prof_short(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                     float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3)
                    for r in _prof_csv(stats_dir, "kernel_stats.csv")), reverse=True)
    kt = ["# Kernel durations of the default bench run, rocprofv3 on MI355X (gfx950)", "#",
          "# commands (from the repository root, after `export TMPDIR=/tmp`):",
          f"#   {PROF_STATS_CMD}", f"#   {PROF_SUM_CMD}", "#",
          f"# {'kernel':78s} {'calls':>7s} {'avg_us':>12s} {'min_us':>12s} {'max_us':>12s} {'pct':>8s}"]
    for pct, name, calls, avg, mn, mx in lines:
        kt.append(f"{name[:80]:80s} {calls:7d} {avg:12.2f} {mn:12.2f} {mx:12.2f} {pct:8.4g}")
    tr = sorted(_prof_csv(stats_dir, "kernel_trace.csv"), key=lambda r: int(r.get("Dispatch_Id", 0) or 0))
    tcm = _prof_call_means([(_prof_short(r["Kernel_Name"]), _prof_grid(r),
                             (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3) for r in tr])
    kt += ["", "# per call: each prefill flavour's calls, kernel by kernel in dispatch order (mean over calls)"]
    for kind, (sig, tv, ncalls) in tcm.items():
        parts = " + ".join(f"{s.split('<')[0]} {t:.1f}" for (s, _), t in zip(sig, tv))
        kt.append(f"{kind:24s} {ncalls:3d} calls  {sum(tv):9.1f} us per call = {parts}")
    with open(os.path.join(out_dir, "kernel_stats_default_bench.txt"), "w") as fh:
        fh.write("\n".join(kt) + "\n")

    ht = ["# HBM traffic per dispatch from rocprofv3 hardware counters, MI355X (gfx950)", "#",
          "# commands (from the repository root, after `export TMPDIR=/tmp`), one counter per run:",
          "#   " + PROF_PMC_CMD.format(c="FETCH_SIZE", d="fetch"),
          "#   " + PROF_PMC_CMD.format(c="WRITE_SIZE", d="write"),
          f"#   {PROF_SUM_CMD}",
          "# sources: gpurun_out/pmc_{fetch,write}/bench_counter_collection.csv (KiB per dispatch)", "#",
          f"# calibration: the same runs copy a {PROFILE_COPY_BYTES:,}-byte buffer (torch copy_, {cw[1]});",
          f"#   that copy reads FETCH_SIZE {cf:.1f} KiB and WRITE_SIZE {cw[0]:.1f} KiB, so FETCH_SIZE is scaled by",
          f"#   {fs:.4f} and WRITE_SIZE by {wsc:.4f} to give bytes moved to or from HBM.",
          "# FETCH_SIZE counts L2 misses, whether the last-level cache (MALL) or HBM serves them: equal",
          "#   counts for a step on one state and on two alternating states say nothing about where they hit.",
          "#",
          f"# per kernel{'':60s} {'grid':>10s} {'FETCH_KiB':>12s} {'WRITE_KiB':>12s} {'HBM_MB':>10s} {'disp':>6s}"]
    for key in sorted(fm):
        if is_m3(fullname[key]):
            b, f, w, n = hbm(key)
            ht.append(f"{key[0][:70]:70s} {key[1]:10d} {f:12.1f} {w:12.1f} {b / 1e6:10.1f} {n:6d}")
    ht.append("")
    for kind, (tot, sig, per_k, ncalls) in call_bytes.items():
        ht.append(f"{kind} ({ncalls} calls): " + " + ".join(f"{k_.split('<')[0]} {b_ / 1e6:.1f}"
                                                           for k_, _, _, b_ in per_k) + f" = {tot / 1e6:.1f} MB")
    ht.append("")
    for tag in list(tags) + list(call_bytes):
        e = K.get(tag)
        if e:
            r, alg = e.get("traffic_over_algorithmic"), e.get("algorithmic_bytes")
            extra = "" if r is None else f"  ({r:.4f}x the algorithmic {alg / 1e6:.1f} MB)"
            ht.append(f"{tag:26s} {e['hbm_bytes_per_launch'] / 1e6:10.1f} MB per launch{extra}")
    ht += ["",
           "# per-call lines: each prefill flavour's calls, kernel by kernel in dispatch order (mean over calls)",
           "# algorithmic bytes (each input read once, outputs written once, the state read and written once):",
           "#   from the bench run's workloads; prefill kernels also carry the chunk-state workspace traffic",
           "#   (written by k_chunk_state, read and rewritten by k_state_pass, read by k_chunk_output) and",
           "#   k_chunk_state re-reads x, B and theta."]
    with open(os.path.join(out_dir, "hbm_counters_default_bench.txt"), "w") as fh:
        fh.write("\n".join(ht) + "\n")


def summarize_sq(sq1_dir, sq2_dir, out_dir, kind="prefill"):
    """mfma_valu_prefill_backward.txt (kind "prefill") or
    mfma_valu_mimo_decode.txt (kind "decode") from two SQ counter runs of the
    prefill and backward workloads, or of the rank-4 decode workloads (one
    step, four tokens per call).  The prefill kernels' MFMAs are bf16
    16x16x32, priced at the dense bf16 peak; the decode kernels' are fp32
    16x16x4, priced at the dense fp32 matrix peak."""
    dec = kind == "decode"
    flops, peak = (MFMA_F32_FLOPS, MFMA_F32_PEAK_TFLOPS) if dec else (MFMA_BF16_FLOPS, MFMA_PEAK_TFLOPS)
    args, sum_flag = (SQ_ARGS_DECODE, "--summarize-sq-decode") if dec else (SQ_ARGS, "--summarize-sq")
    tag = "D" if dec else "M"
    def counters(d):
        acc = {}
        for r in _prof_csv(d, "counter_collection.csv"):
            n = _prof_short(r["Kernel_Name"])
            if n.startswith("k_"):
                acc.setdefault(n, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        return {n: {c: sum(v) / len(v) for c, v in cs.items()} for n, cs in acc.items()}

    c1, c2 = counters(sq1_dir), counters(sq2_dir)
    times = {}
    for r in _prof_csv(sq1_dir, "kernel_trace.csv"):
        times.setdefault(_prof_short(r["Kernel_Name"]), []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    rows = []
    for n, c in c1.items():
        t = sum(times[n]) / len(times[n]) if times.get(n) else float("nan")
        mf, va, lds = c.get("SQ_INSTS_MFMA", 0.0), c.get("SQ_INSTS_VALU", 0.0), c.get("SQ_INSTS_LDS", 0.0)
        mfma_ms = mf * flops / (peak * 1e12) * 1e3
        valu_ms = va * 4 / (1024 * 2.4e9) * 1e3
        conf = c2.get(n, {}).get("SQ_LDS_BANK_CONFLICT", float("nan"))
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        rows.append((t, n, mf, mfma_ms, mfma_ms / (t / 1e3) if t == t else 0.0, va, valu_ms,
                     valu_ms / (t / 1e3) if t == t else 0.0, conf / lds if lds else 0.0, busy / mf if mf else 0.0))
    rows.sort(reverse=True)
    cmd = "rocprofv3 {k}--pmc {s} -f csv -d gpurun_out/pmc{t}{i} -o run -- python3 bench.py " + args
    if dec:
        what = "the rank-4 decode kernels (one step; four tokens per call in group form)"
        pricing = [f"# mfma_ms: the executed MFMA work (SQ_INSTS_MFMA x {flops} flops for v_mfma_f32_16x16x4_f32,",
                   "#   i.e. 16 x 16 x 4 multiply-adds at 2 flops each) at the dense fp32 matrix peak of",
                   "#   157.3 TFLOP/s; mfma_use = mfma_ms / time."]
    else:
        what = "the prefill and backward kernels"
        pricing = [f"# mfma_ms: the executed MFMA work (SQ_INSTS_MFMA x {flops} flops for "
                   "v_mfma_f32_16x16x32_bf16, i.e.",
                   "#   16 x 16 x 32 multiply-adds at 2 flops each, hi/lo operand splits included) at the dense bf16",
                   "#   peak of 2.5 PFLOP/s; mfma_use = mfma_ms / time.",
                   "#   SQ_VALU_MFMA_BUSY_CYCLES reads 16 per such instruction in every kernel (busy/mfma)."]
    txt = [f"# Matrix-core (MFMA) and VALU use of {what}, MI355X (gfx950)", "#",
           "# commands (from the repository root, after `export TMPDIR=/tmp`), one counter set per run:",
           "#   " + cmd.format(k="--kernel-trace ", s=SQ_SETS[0], t=tag, i=1),
           "#   " + cmd.format(k="", s=SQ_SETS[1], t=tag, i=2),
           f"#   python3 bench.py {sum_flag} gpurun_out/pmc{tag}1 gpurun_out/pmc{tag}2",
           "# per dispatch, mean over the dispatches of the run; time_us = the kernel-trace durations of the",
           "#   first run (kernels serialised by the counter collection).", "#"] + pricing + [
           "# valu_ms: SQ_INSTS_VALU at one wave64 instruction per 4 cycles per SIMD (1024 SIMDs, 2.4 GHz);",
           "#   valu_use = valu_ms / time.  The two pipes run side by side (different waves), so the uses do",
           "#   not add up.",
           "# lds_conf: SQ_LDS_BANK_CONFLICT cycles per LDS instruction."] + ([] if dec else [
           "# k_chunk_state and k_state_pass at a single input appear at both chunk lengths (the forward at 128",
           "#   tokens, the backward's recomputed states at 64); rows of one name and template are merged."]) + ["",
           f"{'kernel':70s} {'time_us':>8s} {'MFMA_inst':>10s} {'mfma_ms':>8s} {'mfma_use':>8s} {'VALU_inst':>10s} "
           f"{'valu_ms':>8s} {'valu_use':>8s} {'lds_conf':>8s} {'busy/mfma':>9s}"]
    for t, n, mf, mms, mu, va, vms, vu, lc, bpm in rows:
        txt.append(f"{n[:70]:70s} {t:8.1f} {mf:10.3g} {mms:8.3f} {mu:8.3f} {va:10.4g} {vms:8.3f} {vu:8.3f} "
                   f"{lc:8.3f} {bpm:9.1f}")
    name = "mfma_valu_mimo_decode.txt" if dec else "mfma_valu_prefill_backward.txt"
    with open(os.path.join(out_dir, name), "w") as fh:
        fh.write("\n".join(txt) + "\n")


# ---------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default="", help="comma list of workloads to run (default all)")
    ap.add_argument("--summarize-profiles", nargs=4, metavar=("STATS_DIR", "FETCH_DIR", "WRITE_DIR", "BENCH_JSON"),
                    help="write the rocprofv3 summaries under profiles/ from a profiled run's CSV files and exit")
    ap.add_argument("--summarize-sq", nargs=2, metavar=("SQ1_DIR", "SQ2_DIR"),
                    help="write the MFMA/VALU summary under profiles/ from two SQ counter runs and exit")
    ap.add_argument("--summarize-sq-decode", nargs=2, metavar=("SQ1_DIR", "SQ2_DIR"),
                    help="the same for the rank-4 decode kernels' SQ counter runs")
    ap.add_argument("--profiles-out", default=os.path.join(ROOT, "profiles"),
                    help="directory the summaries go to (default: profiles/)")
    a = ap.parse_args()
    if a.summarize_profiles or a.summarize_sq or a.summarize_sq_decode:   # no GPU needed
        if a.summarize_profiles:
            summarize_profiles(*a.summarize_profiles, a.profiles_out)
        if a.summarize_sq:
            summarize_sq(*a.summarize_sq, a.profiles_out)
        if a.summarize_sq_decode:
            summarize_sq(*a.summarize_sq_decode, a.profiles_out, kind="decode")
        return
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
    # the same steps alternating between two states (537 MB, more than the
    # last-level cache): what a model with several layers sees
    cold = {}
    for name in ("siso_decode", "mimo_decode"):
        if want(name + "_cold"):
            cold[name] = bench_decode(name, a.steps, a.warmup, cold=True)
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
        # every host thread, then one thread on a smaller sample
        if "siso_decode" in res:
            cpu["siso_decode"] = with_single_thread(cpu_decode("siso_decode", 6.0),
                                                    cpu_decode("siso_decode", 3.0, 1, nb=2))
        if "mimo_decode" in res:
            cpu["mimo_decode"] = with_single_thread(cpu_decode("mimo_decode", 5.0),
                                                    cpu_decode("mimo_decode", 3.0, 1, nb=2))
        if "siso_prefill" in res:
            cpu["siso_prefill"] = with_single_thread(
                cpu_prefill("siso_prefill", heads=8, tokens=2048),
                cpu_prefill("siso_prefill", heads=4, tokens=2048, nthreads=1))
        if "mimo_prefill" in res:
            cpu["mimo_prefill"] = with_single_thread(
                cpu_prefill("mimo_prefill", heads=4, tokens=4096),
                cpu_prefill("mimo_prefill", heads=2, tokens=4096, nthreads=1))
        log(f"cpu baselines took {time.time() - t0:.1f}s")

    def decode_entry(r, tag):
        w = r["workload"]
        gbs = r["bytes"] / (r["step_ms"] * 1e-3) / 1e9
        traffic = counters_for(tag) if r["states"] == 1 else None
        sp = r["spread"]
        return dict(
            us_per_step=round(r["step_ms"] * 1e3, 2), us_per_step_spread=sp,
            stream_launch_us_per_step=round(r["stream_step_ms"] * 1e3, 2),
            hbm_gbs=round(gbs, 1), tokens_per_s=round(w.batch / (r["step_ms"] * 1e-3), 1),
            algorithmic_bytes=r["bytes"], input_pool=r["pool"], states=r["states"],
            roofline=dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                          frac=round(gbs / HBM_PEAK_GBS, 4), traffic=traffic,
                          kernel=f"k_decode_{'siso' if w.rank == 1 else 'mimo'}",
                          timing=f"HIP events around each of {sp['replays']} replays of a graph "
                                 f"of the K launches (one kernel per step); median replay"),
            cpu_baseline=cpu.get(tag))

    def prefill_entry(r, tag):
        ach = r["bytes"] / (r["call_ms"] * 1e-3) / 1e9
        if "nseq" in r:   # packed sequences: no separate counters or CPU leg
            return dict(
                ms_per_call=round(r["call_ms"], 4), p50_ms=round(r["call_p50_ms"], 4),
                tokens_per_s=round(r["tokens"] / (r["call_ms"] * 1e-3), 1),
                sequences=r["nseq"], lengths=r["lengths"], algorithmic_bytes=r["bytes"],
                workspace_bytes=r["ws_bytes"], hbm_frac=round(ach / HBM_PEAK_GBS, 4))
        fl = prefill_flops(r["workload"].with_(chunk=r["chunk"]))
        tf = fl / (r["call_ms"] * 1e-3) / 1e12
        return dict(
            ms_per_call=round(r["call_ms"], 4), p50_ms=round(r["call_p50_ms"], 4),
            chunk=r["chunk"],
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
    for base, r in cold.items():
        e = decode_entry(r, base + "_cold")
        e.pop("cpu_baseline")
        if base in workloads:
            e["step_time_vs_cache_warm"] = round(e["us_per_step"] / workloads[base]["us_per_step"], 3)
        workloads[base + "_cold"] = e
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
    for sfx in ("", "_cold"):   # ratios of the median replays
        if "mimo_decode" + sfx in workloads and "siso_decode" + sfx in workloads:
            workloads["mimo_decode" + sfx]["step_time_vs_siso"] = round(
                workloads["mimo_decode" + sfx]["us_per_step"]
                / workloads["siso_decode" + sfx]["us_per_step"], 3)
    line["workloads"] = workloads
    if copy_ref is not None:
        line["hbm_copy_reference"] = copy_ref
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
