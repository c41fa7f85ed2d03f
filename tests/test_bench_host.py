"""Host-side logic of bench.py: the algorithmic byte counts it prices the
roofline with, the one-GPU guard, and the rocprofv3 summaries it writes
under profiles/ (run here on small synthetic CSV files)."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from linear_recurrent_sequence_mamba_amd import inputs as I  # noqa: E402


def test_decode_bytes_headline():
    # state read and written once (fp32), x and x_prev, B_t, B_{t-1}, C_t,
    # dt, lam, theta (bf16), A (fp32 per head), y (fp32)
    w = I.WORKLOADS["siso_decode"]
    B, H, P, N = 128, 64, 64, 128
    assert (w.batch, w.nheads, w.headdim, w.dstate, w.rank) == (B, H, P, N, 1)
    state = 2 * B * H * P * N * 4
    ins = 2 * (2 * B * H * P + 3 * B * H * N + 2 * B * H + B * H * N // 2)
    assert bench.decode_bytes(w) == state + ins + 4 * H + 4 * B * H * P == 548_438_272


def test_prefill_bytes_siso():
    w = I.WORKLOADS["siso_prefill"]
    B, T, H, P, N = 4, 2048, 32, 64, 128
    assert (w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.rank) == (B, T, H, P, N, 1)
    ins = 2 * (B * T * H * P + 2 * B * T * H * N + 2 * B * T * H + B * T * H * N // 2)
    assert bench.prefill_bytes(w) == ins + B * H * P * N * 4 + 4 * H + 4 * B * T * H * P == 273_678_464


def test_more_than_one_gpu_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def _write(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=list(rows[0]))
        wr.writeheader()
        wr.writerows(rows)


DEC = "void m3::(anonymous namespace)::k_decode_siso<m3::bf16_t, float, 128, true, false, false>(m3::DecodeArgs)"
K1 = "void m3::(anonymous namespace)::k_chunk_state<m3::PolB16, m3::bf16_t, 64, 128, 1, false, 128>(m3::PrefillArgs)"
K2 = "void m3::(anonymous namespace)::k_state_pass<m3::bf16_t, 128, 1>(m3::PassArgs)"
K3 = ("void m3::(anonymous namespace)::k_chunk_output<m3::PolB16, m3::bf16_t, float, 64, 128, 1, false, 128>"
      "(m3::PrefillArgs)")
COPY = "__amd_rocclr_copyBuffer"


def _dispatches():
    """(kernel, grid, FETCH KiB, WRITE KiB, duration ns): a device copy of
    256 MiB, two decode steps, two prefill calls of three kernels."""
    d = [(COPY, 1000, 131072.0, 262144.0, 50000)]
    d += [(DEC, 2097152, 262144.0, 266000.0, 88000)] * 2
    for _ in range(2):
        d += [(K1, 1048576, 100.0, 50.0, 68000), (K2, 262144, 70.0, 70.0, 25000),
              (K3, 1048576, 150.0, 60.0, 107000)]
    return d


def _profile_dirs(tmp):
    d = _dispatches()
    for name, col in (("fetch", 2), ("write", 3)):
        cname = "FETCH_SIZE" if name == "fetch" else "WRITE_SIZE"
        _write(os.path.join(tmp, name, "x", "bench_counter_collection.csv"),
               [dict(Dispatch_Id=i + 1, Kernel_Name=r[0], Grid_Size=r[1], Counter_Name=cname,
                     Counter_Value=r[col]) for i, r in enumerate(d)])
    t0 = 0
    trace = []
    for i, r in enumerate(d):
        trace.append(dict(Dispatch_Id=i + 1, Kernel_Name=r[0], Grid_Size=r[1], Start_Timestamp=t0,
                          End_Timestamp=t0 + r[4]))
        t0 += r[4] + 1000
    _write(os.path.join(tmp, "stats", "x", "bench_kernel_trace.csv"), trace)
    names = sorted(set(r[0] for r in d))
    tot = sum(r[4] for r in d)
    _write(os.path.join(tmp, "stats", "x", "bench_kernel_stats.csv"),
           [dict(Name=n, Calls=sum(r[0] == n for r in d), AverageNs=sum(r[4] for r in d if r[0] == n)
                 / sum(r[0] == n for r in d), MinNs=min(r[4] for r in d if r[0] == n),
                 MaxNs=max(r[4] for r in d if r[0] == n),
                 Percentage=100.0 * sum(r[4] for r in d if r[0] == n) / tot) for n in names])
    bj = os.path.join(tmp, "bench.json")
    with open(bj, "w") as fh:
        fh.write("log line\n" + json.dumps({"workloads": {
            "siso_decode": {"algorithmic_bytes": 548_438_272},
            "siso_prefill": {"algorithmic_bytes": 273_678_464}}}) + "\n")
    return [os.path.join(tmp, x) for x in ("stats", "fetch", "write")] + [bj]


def test_summarize_profiles(tmp_path):
    out = tmp_path / "profiles"
    out.mkdir()
    bench.summarize_profiles(*_profile_dirs(str(tmp_path)), str(out))
    data = json.loads((out / "hbm_counters.json").read_text())
    # the 256 MiB copy fixes the scales: FETCH x 2, WRITE x 1
    assert data["fetch_scale"] == 2.0 and data["write_scale"] == 1.0
    dec = data["kernels"]["siso_decode"]
    assert dec["hbm_bytes_per_launch"] == round((2 * 262144.0 + 266000.0) * 1024)
    assert dec["source_hash"] == bench.source_hash(dec["sources"])
    assert dec["traffic_over_algorithmic"] == round(dec["hbm_bytes_per_launch"] / 548_438_272, 4)
    call = data["kernels"]["siso_prefill"]
    assert call["calls"] == 2
    assert [k["kernel"].split("<")[0] for k in call["per_kernel"]] == \
        ["k_chunk_state", "k_state_pass", "k_chunk_output"]
    assert call["hbm_bytes_per_launch"] == round(((100 + 70 + 150) * 2 + (50 + 70 + 60)) * 1024)
    stats = (out / "kernel_stats_default_bench.txt").read_text()
    assert "bench.py --summarize-profiles" in stats
    assert "siso_prefill" in stats and "200.0 us per call" in stats
    hbm = (out / "hbm_counters_default_bench.txt").read_text()
    assert "rocprofv3 --pmc FETCH_SIZE" in hbm and "scaled by" in hbm


def test_summarize_cli_needs_no_gpu(tmp_path):
    dirs = _profile_dirs(str(tmp_path))
    out = tmp_path / "out"
    out.mkdir()
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--summarize-profiles", *dirs,
                        "--profiles-out", str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert sorted(os.listdir(out)) == ["hbm_counters.json", "hbm_counters_default_bench.txt",
                                       "kernel_stats_default_bench.txt"]


@pytest.mark.parametrize("name, short", [
    (K3, "k_chunk_output<PolB16, bf16_t, float, 64, 128, 1, false, 128>"),
    ("void at::native::f<4, g<float>>(int, h<(i)>)", "at::native::f<4, g<float>>"),
])
def test_kernel_short_names(name, short):
    assert bench._prof_short(name) == short


def _sq_dirs(tmp, kernel, mfma, valu, lds, conflicts, dur_ns):
    """Two SQ counter runs (and the first run's kernel trace) of one dispatch."""
    sq1, sq2 = os.path.join(tmp, "sq1"), os.path.join(tmp, "sq2")
    vals = {"SQ_INSTS_MFMA": mfma, "SQ_INSTS_VALU": valu, "SQ_INSTS_LDS": lds}
    _write(os.path.join(sq1, "x", "run_counter_collection.csv"),
           [dict(Dispatch_Id=1, Kernel_Name=kernel, Grid_Size=1, Counter_Name=c, Counter_Value=vals.get(c, 1.0))
            for c in bench.SQ_SETS[0].split()])
    _write(os.path.join(sq1, "x", "run_kernel_trace.csv"),
           [dict(Dispatch_Id=1, Kernel_Name=kernel, Grid_Size=1, Start_Timestamp=0, End_Timestamp=dur_ns)])
    _write(os.path.join(sq2, "x", "run_counter_collection.csv"),
           [dict(Dispatch_Id=1, Kernel_Name=kernel, Grid_Size=1, Counter_Name=c,
                 Counter_Value=conflicts if c == "SQ_LDS_BANK_CONFLICT" else 1.0)
            for c in bench.SQ_SETS[1].split()])
    return sq1, sq2


@pytest.mark.parametrize("kind", ["prefill", "decode"])
def test_summarize_sq(tmp_path, kind):
    """The decode kernels' MFMAs (fp32 16x16x4) are priced at the fp32 matrix
    peak, the prefill kernels' (bf16 16x16x32) at the bf16 peak."""
    kern = ("void m3::k_decode_mimo_grp<m3::bf16_t, float, 128, true, false, true>(m3::DecodeArgs)"
            if kind == "decode" else K3)
    dirs = _sq_dirs(str(tmp_path), kern, mfma=1e9, valu=2e8, lds=1000.0, conflicts=500.0, dur_ns=1_000_000)
    out = tmp_path / "out"
    out.mkdir()
    bench.summarize_sq(*dirs, str(out), kind=kind)
    name = "mfma_valu_mimo_decode.txt" if kind == "decode" else "mfma_valu_prefill_backward.txt"
    txt = (out / name).read_text()
    row = [ln for ln in txt.splitlines() if ln.startswith(bench._prof_short(kern)[:60])]
    assert len(row) == 1
    f = row[0][70:].split()
    flops, peak = ((2 * 16 * 16 * 4, 157.3) if kind == "decode" else (2 * 16 * 16 * 32, 2500.0))
    mfma_ms = 1e9 * flops / (peak * 1e12) * 1e3
    assert float(f[0]) == pytest.approx(1000.0)                      # time_us
    assert float(f[2]) == pytest.approx(mfma_ms, abs=1e-3)            # mfma_ms
    assert float(f[3]) == pytest.approx(mfma_ms / 1.0, abs=2e-3)      # use over 1 ms
    assert float(f[7]) == pytest.approx(0.5)                          # conflict cycles per LDS instruction
    flag = "--summarize-sq-decode" if kind == "decode" else "--summarize-sq "
    assert flag in txt
