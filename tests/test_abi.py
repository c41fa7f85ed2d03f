"""Host-only checks of the C ABI: the library loads, exports every function
that include/m3ssm.h declares, and rejects bad arguments before launching
anything (no GPU needed: every call here fails its host-side checks)."""
import ctypes
import os
import re

import pytest

from linear_recurrent_sequence_mamba_amd import binding as m3

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "m3ssm.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_ ]*[\s\*]+(m3_[a-z_]+)\s*\(",
                                 src, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("m3_scan_prefill", "m3_scan_prefill_varlen", "m3_scan_prefill_backward",
              "m3_prefill_backward_workspace_size", "m3_decode_step",
              "m3_decode_tokens", "m3_prefill_workspace_size",
              "m3_prefill_varlen_workspace_size", "m3_status_str", "m3_last_hip_error"):
        assert n in names, names


def test_library_exports_every_declared_symbol():
    lib = m3.library()
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_status_strings():
    for s in range(9):
        assert m3.m3_status_str(s) != "unknown status"
    assert m3.m3_status_str(99) == "unknown status"


def _dims(**kw):
    base = dict(batch=2, seqlen=100, nheads=3, headdim=64, dstate=128, rank=1, chunk=0,
                in_dtype=m3.M3_BF16, out_dtype=m3.M3_F32, flags=0, ngroups=0)
    base.update(kw)
    return m3.m3_dims(*base.values())


P16 = ctypes.c_void_p(4096)   # a 16-byte aligned non-NULL address that is never dereferenced
P_MIS = ctypes.c_void_p(4100)


def _decode(d, **over):
    args = dict(h=P16, x=P16, xp=None, Bt=P16, Bp=None, C=P16, dt=P16, A=P16, lam=P16, th=P16, y=P16)
    args.update(over)
    return m3.library().m3_decode_step(ctypes.byref(d), *args.values(), None)


def _tokens(d, **over):
    args = dict(h=P16, x=P16, xp=None, Bt=P16, Bp=None, C=P16, dt=P16, A=P16, lam=P16, th=P16, y=P16)
    args.update(over)
    return m3.library().m3_decode_tokens(ctypes.byref(d), *args.values(), None)


def _prefill(d, ws_bytes=1 << 40, **over):
    args = dict(x=P16, dt=P16, A=P16, lam=P16, th=P16, B=P16, C=P16, h0=None, xp=None, Bp=None,
                y=P16, hT=None, ws=P16)
    args.update(over)
    return m3.library().m3_scan_prefill(ctypes.byref(d), *args.values(), ws_bytes, None)


def _noalloc(d, **over):
    args = dict(x=P16, dt=P16, A=P16, lam=P16, th=P16, B=P16, C=P16, h0=None, xp=None, Bp=None,
                y=P16, hT=None)
    args.update(over)
    return m3.library().m3_scan_prefill_noalloc(ctypes.byref(d), *args.values(), None)


def _varlen(d, ws_bytes=1 << 40, **over):
    args = dict(cu=P16, x=P16, dt=P16, A=P16, lam=P16, th=P16, B=P16, C=P16, h0=None, xp=None,
                Bp=None, y=P16, hT=None, ws=P16)
    args.update(over)
    return m3.library().m3_scan_prefill_varlen(ctypes.byref(d), *args.values(), ws_bytes, None)


def _backward(d, ws_bytes=1 << 40, **over):
    args = dict(x=P16, dt=P16, A=P16, lam=P16, th=P16, B=P16, C=P16, h0=None, xp=None, Bp=None,
                dy=P16, dhT=None, gx=P16, gdt=P16, gA=P16, glam=P16, gth=P16, gB=P16, gC=P16,
                gh0=None, gxp=None, gBp=None, ws=P16)
    args.update(over)
    return m3.library().m3_scan_prefill_backward(ctypes.byref(d), *args.values(), ws_bytes, None)


def test_workspace_size():
    # one P x N state per chunk: a single input takes 128-token chunks by
    # default, 64-token ones when asked
    d = _dims(batch=4, seqlen=2048, nheads=32)
    n = m3.m3_prefill_workspace_size(d)
    assert 4 * 32 * 16 * 64 * 128 * 4 <= n < 4 * 32 * 17 * 64 * 128 * 4
    n64 = m3.m3_prefill_workspace_size(_dims(batch=4, seqlen=2048, nheads=32, chunk=64))
    assert 4 * 32 * 32 * 64 * 128 * 4 <= n64 < 4 * 32 * 33 * 64 * 128 * 4
    assert m3.m3_prefill_workspace_size(_dims(rank=4)) == \
        m3.m3_prefill_workspace_size(_dims(rank=4, chunk=64))
    assert m3.m3_prefill_workspace_size(_dims(dstate=7)) == 0
    assert m3.library().m3_prefill_workspace_size(None) == 0


@pytest.mark.parametrize("call", [_decode, _tokens, _prefill, _noalloc, _varlen, _backward])
def test_error_paths(call):
    assert m3.library().m3_decode_step(None, *([None] * 12)) == 1
    assert call(_dims(), x=None) == 1                           # NULL input
    assert call(_dims(), xp=P16) == 1                           # x_prev without B_prev
    assert call(_dims(dstate=127)) == 2                         # odd N
    assert call(_dims(headdim=0)) == 2
    assert call(_dims(batch=0)) == 2                            # empty batch
    assert call(_dims(nheads=0)) == 2
    if call is not _decode:
        assert call(_dims(seqlen=0)) == 2                       # no tokens
    assert call(_dims(rank=0)) == 2
    assert call(_dims(flags=1 << 7)) == 2                       # unknown flag
    assert call(_dims(ngroups=-1)) == 2                         # head groups
    assert call(_dims(ngroups=4)) == 2                          # more groups than heads
    assert call(_dims(ngroups=2)) == 2                          # 2 does not divide 3 heads
    assert call(_dims(in_dtype=5)) == 3
    assert call(_dims(out_dtype=-1)) == 3
    assert call(_dims(headdim=24, dstate=6)) == 4               # no kernel for it
    assert call(_dims(), x=P_MIS) == 5                          # misaligned


def test_tokens_specific_errors():
    assert _tokens(_dims(seqlen=0)) == 2                        # no tokens
    assert _tokens(_dims(dstate=24)) == 4                       # no kernel for N = 24
    assert _tokens(_dims(rank=4, headdim=128)) == 4             # MIMO: P <= 64


def test_prefill_specific_errors():
    assert _prefill(_dims(seqlen=0)) == 2
    assert _prefill(_dims(chunk=-1)) == 2
    assert _prefill(_dims(chunk=32)) == 4
    assert _prefill(_dims(), ws=None) == 6
    need = m3.m3_prefill_workspace_size(_dims())
    assert _prefill(_dims(), ws_bytes=need - 1) == 6
    assert _prefill(_dims(), ws=P_MIS) == 5
    assert _prefill(_dims(), hT=P_MIS) == 5


def test_noalloc_specific_errors():
    """Calls whose workspace would exceed the library's scratch buffer are
    refused before anything is looked up or launched."""
    assert _noalloc(_dims(seqlen=0)) == 2
    assert _noalloc(_dims(chunk=32)) == 4
    big = _dims(batch=4, seqlen=2048, nheads=32)
    assert m3.m3_prefill_workspace_size(big) > m3.M3_NOALLOC_SCRATCH_BYTES
    assert _noalloc(big) == 8
    assert _noalloc(big, hT=P_MIS) == 5


def test_varlen_specific_errors():
    assert _varlen(_dims(), cu=None) == 1
    assert _varlen(_dims(), cu=ctypes.c_void_p(4098)) == 5      # offsets are int32
    assert _varlen(_dims(seqlen=0)) == 2
    assert _varlen(_dims(chunk=32)) == 4
    assert _varlen(_dims(), ws=None) == 6
    need = m3.m3_prefill_varlen_workspace_size(_dims())
    assert _varlen(_dims(), ws_bytes=need - 1) == 6


def test_backward_specific_errors():
    assert _backward(_dims(), gx=None) == 1                     # a gradient output is required
    assert _backward(_dims(), dy=None) == 1
    assert _backward(_dims(rank=3)) == 4                        # ranks 1, 2 and 4 only
    assert _backward(_dims(rank=2, headdim=32, dstate=64)) == 4  # R = 2 only with (64, 128)
    assert _backward(_dims(seqlen=0)) == 2
    assert _backward(_dims(), ws=None) == 6
    need = m3.m3_prefill_backward_workspace_size(_dims())
    assert need > m3.m3_prefill_workspace_size(_dims())
    assert _backward(_dims(), ws_bytes=need - 1) == 6
    d = _dims()
    ok = m3.m3_bc_prep(None, None, None, None, 1e-6, 1)
    d.bc = ctypes.pointer(ok)
    assert _backward(d) == 4                                    # no B/C preparation


def test_theta_proj_errors():
    """The angle projection: width a positive multiple of 32, both arrays
    given and aligned; not offered by the multi-token decode or the backward."""
    def with_tp(dim=64, u=P16, W=P16):
        d = _dims()
        tp = m3.m3_theta_proj(u, W, dim)
        d._keep = tp
        d.tp = ctypes.pointer(tp)
        return d
    for call in (_decode, _prefill, _noalloc, _varlen):
        assert call(with_tp(dim=48)) == 2                       # not a multiple of 32
        assert call(with_tp(dim=0)) == 2
        assert call(with_tp(u=None)) == 1
        assert call(with_tp(W=P_MIS)) == 5
        assert call(_dims(), th=None) == 1                      # theta needed without it
    assert _tokens(with_tp()) == 4
    assert _backward(with_tp()) == 4


def test_varlen_workspace_size():
    # S sequences over T tokens take at most min(T, (T + 63 S) / 64) chunks;
    # the per-chunk state (P N fp32) dominates the workspace
    for Q in (64, 128):
        for S, T in ((1, 100), (7, 100), (300, 100), (5, 64 * 40)):
            d = _dims(batch=S, seqlen=T, nheads=3, chunk=Q)
            slots = min(T, (T + (Q - 1) * S) // Q)
            n = m3.m3_prefill_varlen_workspace_size(d)
            assert 3 * slots * 64 * 128 * 4 <= n <= 3 * slots * (64 * 128 + 129) * 4 + 16 * (S + slots) + 1280
    assert m3.m3_prefill_varlen_workspace_size(_dims(dstate=7)) == 0
    # one sequence needs as many chunks as the dense call
    assert m3.m3_prefill_varlen_workspace_size(_dims(batch=1)) >= \
        m3.m3_prefill_workspace_size(_dims(batch=1))


def test_bc_prep_errors():
    for call in (_decode, _tokens, _prefill, _varlen):
        bad_eps = m3.m3_bc_prep(None, None, None, None, -1.0, 1)
        d = _dims()
        d.bc = ctypes.pointer(bad_eps)
        assert call(d) == 2                                     # eps < 0
        nan_eps = m3.m3_bc_prep(None, None, None, None, float("nan"), 1)
        d.bc = ctypes.pointer(nan_eps)
        assert call(d) == 2
        mis = m3.m3_bc_prep(P16, P_MIS, None, None, 1e-6, 1)
        d.bc = ctypes.pointer(mis)
        assert call(d) == 5                                     # misaligned weight
    # the prefill workspace grows by the chunk's B inverse RMS (Q R floats per chunk)
    d = _dims(rank=4)
    plain = m3.m3_prefill_workspace_size(d)
    ok = m3.m3_bc_prep(None, None, None, None, 1e-6, 1)
    d.bc = ctypes.pointer(ok)
    assert m3.m3_prefill_workspace_size(d) >= plain + 2 * 3 * 2 * 64 * 4 * 4
    assert m3.m3_prefill_varlen_workspace_size(d) > m3.m3_prefill_varlen_workspace_size(_dims(rank=4))


def test_binding_rejects_mismatched_tensors():
    torch = pytest.importorskip("torch")
    d = _dims()
    h = torch.zeros(2, 3, 64, 128)  # host tensor: rejected before any call
    with pytest.raises(ValueError):
        m3.m3_decode_step(d, h, *([None] * 10))


def test_missing_library_fails_loudly(monkeypatch):
    """Without the built library every entry point raises: there is no other path."""
    monkeypatch.setattr(m3, "_LIB", None)
    monkeypatch.setattr(m3, "LIB_PATH", "/nonexistent/libm3ssm.so")
    with pytest.raises(RuntimeError, match="is not built"):
        m3.library()
    with pytest.raises(RuntimeError, match="is not built"):
        m3.m3_prefill_workspace_size(_dims())
