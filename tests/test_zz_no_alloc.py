"""m3_scan_prefill_noalloc (the prefill for callers that cannot allocate:
its workspace is the library's own per-GPU scratch buffer) against
m3_scan_prefill with a caller workspace, through the C ABI: equal bits on
two calls in a row, the second one smaller, and sizes beyond the buffer
rejected before anything is launched."""
import ctypes

import pytest
import torch

from linear_recurrent_sequence_mamba_amd import binding as m3
from linear_recurrent_sequence_mamba_amd import inputs as I
from tests.util import cuda, say

pytestmark = pytest.mark.gpu

KEYS = ("x", "dt", "A", "lam", "theta", "B", "C", "h0", "x_prev", "B_prev")


def _both(w, seed):
    d = {k: cuda(v) for k, v in I.prefill_inputs(w, stream=seed, h0="normal",
                                                   with_prev=True).items()}
    dims = m3.make_dims(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.rank, 0,
                        m3.M3_BF16, m3.M3_F32)
    assert m3.m3_prefill_workspace_size(dims) <= m3.M3_NOALLOC_SCRATCH_BYTES
    dev = d["x"].device
    shape_y = (w.batch, w.seqlen, w.nheads, w.headdim, w.rank)
    shape_h = (w.batch, w.nheads, w.headdim, w.dstate)
    y_ref = torch.empty(shape_y, dtype=torch.float32, device=dev)
    h_ref = torch.empty(shape_h, dtype=torch.float32, device=dev)
    ws = m3.workspace(dims, dev)
    m3.m3_scan_prefill(dims, *(d[k] for k in KEYS), y_ref, h_ref, ws)
    y = torch.full(shape_y, float("nan"), device=dev)
    h = torch.full(shape_h, float("nan"), device=dev)
    m3.m3_scan_prefill_noalloc(dims, *(d[k] for k in KEYS), y, h)
    torch.cuda.synchronize()
    return (y, h), (y_ref, h_ref)


@pytest.mark.parametrize("R", [1, 4])
def test_noalloc_equals_workspace_call(R):
    big = I.Workload("na", 140, 2, 1000, 8, 64, 128, R, 64, "bf16")
    small = big.with_(batch=1, seqlen=130, nheads=3)
    for w, seed in ((big, 0), (small, 1)):   # the second call is smaller
        say(f"noalloc prefill R={R} B={w.batch} T={w.seqlen} H={w.nheads}")
        (y, h), (y_ref, h_ref) = _both(w, seed)
        assert torch.equal(y, y_ref) and torch.equal(h, h_ref)


def test_noalloc_rejects_calls_beyond_the_buffer():
    # 4 x 32 heads x 32 chunks of 64 x 128 fp32 states: 128 MiB of workspace
    dims = m3.make_dims(4, 2048, 32, 64, 128, 1, 0, m3.M3_BF16, m3.M3_F32)
    assert m3.m3_prefill_workspace_size(dims) > m3.M3_NOALLOC_SCRATCH_BYTES
    p = ctypes.c_void_p(4096)
    st = m3.library().m3_scan_prefill_noalloc(ctypes.byref(dims), p, p, p, p, p, p, p, None,
                                              None, None, p, None, None)
    assert st == 8 and "scratch" in m3.m3_status_str(st)
