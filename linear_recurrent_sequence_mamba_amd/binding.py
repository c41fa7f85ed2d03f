"""ctypes binding of libm3ssm (include/m3ssm.h).

The functions carry the C names and only marshal arguments: they check that
the torch tensors match the dims (shape, dtype, device, contiguity) so that
no kernel can be handed a buffer smaller than it will touch, then pass the
raw device pointers and the current HIP stream to the library.  All compute
runs in the library's HIP kernels; there is no fallback path.  If the shared
library is missing the first call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libm3ssm.so")

M3_F32, M3_BF16 = 0, 1
M3_THETA_IS_ANGLE = 1 << 0
M3_A_PER_TOKEN = 1 << 1

STATUS = {0: "M3_OK", 1: "M3_ERR_NULL", 2: "M3_ERR_SHAPE", 3: "M3_ERR_DTYPE",
          4: "M3_ERR_UNSUPPORTED", 5: "M3_ERR_ALIGN", 6: "M3_ERR_WORKSPACE", 7: "M3_ERR_HIP",
          8: "M3_ERR_TOO_LARGE"}
M3_NOALLOC_SCRATCH_BYTES = 64 << 20


class m3_bc_prep(ctypes.Structure):
    _fields_ = [("B_weight", ctypes.c_void_p), ("C_weight", ctypes.c_void_p),
                ("B_bias", ctypes.c_void_p), ("C_bias", ctypes.c_void_p),
                ("eps", ctypes.c_float), ("rms", ctypes.c_int32)]


class m3_theta_proj(ctypes.Structure):
    _fields_ = [("u", ctypes.c_void_p), ("W", ctypes.c_void_p), ("dim", ctypes.c_int32)]


class m3_dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32),
                ("nheads", ctypes.c_int32), ("headdim", ctypes.c_int32),
                ("dstate", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("ngroups", ctypes.c_int32), ("bc", ctypes.POINTER(m3_bc_prep)),
                ("tp", ctypes.POINTER(m3_theta_proj))]


class BCPrep:
    """The in-kernel preparation of B and C (m3_bc_prep): RMS normalisation
    over N per rank column, weight [N] and per-head bias [H, N, R], all fp32
    device tensors or None."""

    def __init__(self, B_weight=None, C_weight=None, B_bias=None, C_bias=None, eps=1e-6,
                 rms=True):
        self.B_weight, self.C_weight = B_weight, C_weight
        self.B_bias, self.C_bias = B_bias, C_bias
        self.eps, self.rms = float(eps), bool(rms)

    def struct(self) -> m3_bc_prep:
        return m3_bc_prep(_ptr(self.B_weight), _ptr(self.C_weight), _ptr(self.B_bias),
                          _ptr(self.C_bias), self.eps, int(self.rms))

    def check(self, H, N, R):
        for name in ("B_weight", "C_weight"):
            _check(name, getattr(self, name), (N,), torch.float32, optional=True)
        for name in ("B_bias", "C_bias"):
            _check(name, getattr(self, name), (H, N, R), torch.float32, optional=True)


class ThetaProj:
    """The in-kernel angle projection (m3_theta_proj): theta = W u per token
    row and head group; u [rows..., D] and W [G, N/2, D] device tensors in
    the input dtype."""

    def __init__(self, u, W):
        self.u, self.W = u, W
        self.dim = int(W.shape[-1])

    def struct(self) -> m3_theta_proj:
        return m3_theta_proj(_ptr(self.u), _ptr(self.W), self.dim)

    def check(self, rows, G, N, dtype):
        _check("tp.u", self.u, tuple(rows) + (self.dim,), dtype)
        _check("tp.W", self.W, (G, N // 2, self.dim), dtype)


class M3Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {STATUS.get(status, status)} ({_status_str(status)})"
        if status == 7:
            msg += f", hip error {_lib().m3_last_hip_error()}"
        super().__init__(msg)


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m linear_recurrent_sequence_mamba_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp, sz, dp = ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(m3_dims)
        lib.m3_prefill_workspace_size.restype = sz
        lib.m3_prefill_workspace_size.argtypes = [dp]
        lib.m3_scan_prefill.restype = ctypes.c_int
        lib.m3_scan_prefill.argtypes = [dp] + [vp] * 13 + [sz, vp]
        lib.m3_scan_prefill_noalloc.restype = ctypes.c_int
        lib.m3_scan_prefill_noalloc.argtypes = [dp] + [vp] * 12 + [vp]
        lib.m3_prefill_backward_workspace_size.restype = sz
        lib.m3_prefill_backward_workspace_size.argtypes = [dp]
        lib.m3_scan_prefill_backward.restype = ctypes.c_int
        lib.m3_scan_prefill_backward.argtypes = [dp] + [vp] * 23 + [sz, vp]
        lib.m3_prefill_varlen_workspace_size.restype = sz
        lib.m3_prefill_varlen_workspace_size.argtypes = [dp]
        lib.m3_scan_prefill_varlen.restype = ctypes.c_int
        lib.m3_scan_prefill_varlen.argtypes = [dp] + [vp] * 14 + [sz, vp]
        lib.m3_decode_step.restype = ctypes.c_int
        lib.m3_decode_step.argtypes = [dp] + [vp] * 11 + [vp]
        lib.m3_decode_tokens.restype = ctypes.c_int
        lib.m3_decode_tokens.argtypes = [dp] + [vp] * 11 + [vp]
        lib.m3_status_str.restype = ctypes.c_char_p
        lib.m3_status_str.argtypes = [ctypes.c_int]
        lib.m3_last_hip_error.restype = ctypes.c_int
        lib.m3_last_hip_error.argtypes = []
        _LIB = lib
    return _LIB


def library():
    """The loaded ctypes library (loads it on first use)."""
    return _lib()


def _status_str(s: int) -> str:
    return _lib().m3_status_str(int(s)).decode()


def m3_status_str(status: int) -> str:
    return _status_str(status)


def make_dims(batch, seqlen, nheads, headdim, dstate, rank=1, chunk=0,
              in_dtype=M3_BF16, out_dtype=M3_F32, flags=0, ngroups=0, bc=None,
              tp=None) -> m3_dims:
    """bc: a BCPrep, tp: a ThetaProj (both kept alive by the returned dims)
    or None."""
    d = m3_dims(batch, seqlen, nheads, headdim, dstate, rank, chunk, in_dtype,
                out_dtype, flags, ngroups)
    if bc is not None:
        d._bc_struct = bc.struct()
        d._bc = bc
        d.bc = ctypes.pointer(d._bc_struct)
    if tp is not None:
        d._tp_struct = tp.struct()
        d._tp = tp
        d.tp = ctypes.pointer(d._tp_struct)
    return d


def _check_bc(d: m3_dims):
    bc = getattr(d, "_bc", None)
    if bc is not None:
        bc.check(d.nheads, d.dstate, d.rank)


def _proj(d: m3_dims):
    """The dims' ThetaProj, or None (theta is then a required input)."""
    return getattr(d, "_tp", None)


def groups(d: m3_dims) -> int:
    """B, C and theta groups of a call (ngroups, or nheads when it is 0)."""
    return d.ngroups if d.ngroups > 0 else d.nheads


def dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return M3_BF16
    if t == torch.float32:
        return M3_F32
    raise TypeError(f"unsupported dtype {t}")


_TORCH = {M3_BF16: torch.bfloat16, M3_F32: torch.float32}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(name, t, shape, dtype, optional=False):
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype} != expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def m3_prefill_workspace_size(dims: m3_dims) -> int:
    return int(_lib().m3_prefill_workspace_size(ctypes.byref(dims)))


def m3_scan_prefill(dims: m3_dims, x, dt, A, lam, theta, B, C, h0, x_prev, B_prev,
                    y, hT, ws, stream=None) -> None:
    d = dims
    ti, to = _TORCH.get(d.in_dtype), _TORCH.get(d.out_dtype)
    if ti is not None and to is not None:
        Bsz, T, H, P, N, R = d.batch, d.seqlen, d.nheads, d.headdim, d.dstate, d.rank
        G = groups(d)
        _check("x", x, (Bsz, T, H, P, R), ti)
        _check("dt", dt, (Bsz, T, H), ti)
        _check("A", A, (Bsz, T, H) if d.flags & M3_A_PER_TOKEN else (H,), torch.float32)
        _check("lam", lam, (Bsz, T, H), ti)
        _check("theta", theta, (Bsz, T, G, N // 2), ti, optional=_proj(d) is not None)
        if _proj(d) is not None:
            _proj(d).check((Bsz, T), G, N, ti)
        _check("B", B, (Bsz, T, G, N, R), ti)
        _check("C", C, (Bsz, T, G, N, R), ti)
        _check("h0", h0, (Bsz, H, P, N), torch.float32, optional=True)
        _check("x_prev", x_prev, (Bsz, H, P, R), ti, optional=True)
        _check("B_prev", B_prev, (Bsz, G, N, R), ti, optional=True)
        _check("y", y, (Bsz, T, H, P, R), to)
        _check("hT", hT, (Bsz, H, P, N), torch.float32, optional=True)
    nbytes = 0
    if ws is not None:
        if not ws.is_cuda or not ws.is_contiguous():
            raise ValueError("ws must be a contiguous device tensor")
        nbytes = ws.numel() * ws.element_size()
    _check_bc(d)
    st = _lib().m3_scan_prefill(ctypes.byref(d), _ptr(x), _ptr(dt), _ptr(A), _ptr(lam),
                                _ptr(theta), _ptr(B), _ptr(C), _ptr(h0), _ptr(x_prev),
                                _ptr(B_prev), _ptr(y), _ptr(hT), _ptr(ws), nbytes,
                                _stream(stream))
    if st != 0:
        raise M3Error(st, "m3_scan_prefill")


def m3_scan_prefill_noalloc(dims: m3_dims, x, dt, A, lam, theta, B, C, h0, x_prev, B_prev,
                            y, hT, stream=None) -> None:
    """m3_scan_prefill with the library's own scratch buffer (no workspace
    argument; calls that overlap on one GPU race)."""
    d = dims
    ti, to = _TORCH.get(d.in_dtype), _TORCH.get(d.out_dtype)
    if ti is not None and to is not None:
        Bsz, T, H, P, N, R = d.batch, d.seqlen, d.nheads, d.headdim, d.dstate, d.rank
        G = groups(d)
        _check("x", x, (Bsz, T, H, P, R), ti)
        _check("dt", dt, (Bsz, T, H), ti)
        _check("A", A, (Bsz, T, H) if d.flags & M3_A_PER_TOKEN else (H,), torch.float32)
        _check("lam", lam, (Bsz, T, H), ti)
        _check("theta", theta, (Bsz, T, G, N // 2), ti, optional=_proj(d) is not None)
        if _proj(d) is not None:
            _proj(d).check((Bsz, T), G, N, ti)
        _check("B", B, (Bsz, T, G, N, R), ti)
        _check("C", C, (Bsz, T, G, N, R), ti)
        _check("h0", h0, (Bsz, H, P, N), torch.float32, optional=True)
        _check("x_prev", x_prev, (Bsz, H, P, R), ti, optional=True)
        _check("B_prev", B_prev, (Bsz, G, N, R), ti, optional=True)
        _check("y", y, (Bsz, T, H, P, R), to)
        _check("hT", hT, (Bsz, H, P, N), torch.float32, optional=True)
    _check_bc(d)
    st = _lib().m3_scan_prefill_noalloc(ctypes.byref(d), _ptr(x), _ptr(dt), _ptr(A), _ptr(lam),
                                        _ptr(theta), _ptr(B), _ptr(C), _ptr(h0), _ptr(x_prev),
                                        _ptr(B_prev), _ptr(y), _ptr(hT), _stream(stream))
    if st != 0:
        raise M3Error(st, "m3_scan_prefill_noalloc")


def m3_prefill_backward_workspace_size(dims: m3_dims) -> int:
    return int(_lib().m3_prefill_backward_workspace_size(ctypes.byref(dims)))


GRAD_NAMES = ("x", "dt", "A", "lam", "theta", "B", "C", "h0", "x_prev", "B_prev")


def m3_scan_prefill_backward(dims: m3_dims, x, dt, A, lam, theta, B, C, h0, x_prev, B_prev, dy,
                             dhT, grads: dict, ws, stream=None) -> None:
    """grads: fp32 device tensors keyed by GRAD_NAMES (h0, x_prev, B_prev may
    be missing or None)."""
    d = dims
    ti, to = _TORCH.get(d.in_dtype), _TORCH.get(d.out_dtype)
    if ti is not None and to is not None:
        Bsz, T, H, P, N, R = d.batch, d.seqlen, d.nheads, d.headdim, d.dstate, d.rank
        G = groups(d)
        f32 = torch.float32
        shapes = dict(x=(Bsz, T, H, P, R), dt=(Bsz, T, H), lam=(Bsz, T, H),
                      A=(Bsz, T, H) if d.flags & M3_A_PER_TOKEN else (H,),
                      theta=(Bsz, T, G, N // 2), B=(Bsz, T, G, N, R), C=(Bsz, T, G, N, R),
                      h0=(Bsz, H, P, N), x_prev=(Bsz, H, P, R), B_prev=(Bsz, G, N, R))
        for k, t in (("x", x), ("dt", dt), ("lam", lam), ("theta", theta), ("B", B), ("C", C)):
            _check(k, t, shapes[k], ti)
        _check("A", A, shapes["A"], f32)
        _check("h0", h0, shapes["h0"], f32, optional=True)
        _check("x_prev", x_prev, shapes["x_prev"], ti, optional=True)
        _check("B_prev", B_prev, shapes["B_prev"], ti, optional=True)
        _check("dy", dy, shapes["x"], to)
        _check("dhT", dhT, shapes["h0"], f32, optional=True)
        for k in GRAD_NAMES:
            _check("d" + k, grads.get(k), shapes[k], f32,
                   optional=k in ("h0", "x_prev", "B_prev"))
    nbytes = 0
    if ws is not None:
        if not ws.is_cuda or not ws.is_contiguous():
            raise ValueError("ws must be a contiguous device tensor")
        nbytes = ws.numel() * ws.element_size()
    _check_bc(d)
    gp = lambda k: _ptr(grads.get(k))
    st = _lib().m3_scan_prefill_backward(
        ctypes.byref(d), _ptr(x), _ptr(dt), _ptr(A), _ptr(lam), _ptr(theta), _ptr(B), _ptr(C),
        _ptr(h0), _ptr(x_prev), _ptr(B_prev), _ptr(dy), _ptr(dhT), gp("x"), gp("dt"), gp("A"),
        gp("lam"), gp("theta"), gp("B"), gp("C"), gp("h0"), gp("x_prev"), gp("B_prev"), _ptr(ws),
        nbytes, _stream(stream))
    if st != 0:
        raise M3Error(st, "m3_scan_prefill_backward")


def m3_prefill_varlen_workspace_size(dims: m3_dims) -> int:
    return int(_lib().m3_prefill_varlen_workspace_size(ctypes.byref(dims)))


def m3_scan_prefill_varlen(dims: m3_dims, cu_seqlens, x, dt, A, lam, theta, B, C, h0, x_prev,
                           B_prev, y, hT, ws, stream=None) -> None:
    """Packed sequences: dims.batch = S sequences, dims.seqlen = T total
    tokens; cu_seqlens is a device int32 tensor of S + 1 offsets."""
    d = dims
    ti, to = _TORCH.get(d.in_dtype), _TORCH.get(d.out_dtype)
    if ti is not None and to is not None:
        S, T, H, P, N, R = d.batch, d.seqlen, d.nheads, d.headdim, d.dstate, d.rank
        G = groups(d)
        _check("cu_seqlens", cu_seqlens, (S + 1,), torch.int32)
        _check("x", x, (T, H, P, R), ti)
        _check("dt", dt, (T, H), ti)
        _check("A", A, (T, H) if d.flags & M3_A_PER_TOKEN else (H,), torch.float32)
        _check("lam", lam, (T, H), ti)
        _check("theta", theta, (T, G, N // 2), ti, optional=_proj(d) is not None)
        if _proj(d) is not None:
            _proj(d).check((T,), G, N, ti)
        _check("B", B, (T, G, N, R), ti)
        _check("C", C, (T, G, N, R), ti)
        _check("h0", h0, (S, H, P, N), torch.float32, optional=True)
        _check("x_prev", x_prev, (S, H, P, R), ti, optional=True)
        _check("B_prev", B_prev, (S, G, N, R), ti, optional=True)
        _check("y", y, (T, H, P, R), to)
        _check("hT", hT, (S, H, P, N), torch.float32, optional=True)
    nbytes = 0
    if ws is not None:
        if not ws.is_cuda or not ws.is_contiguous():
            raise ValueError("ws must be a contiguous device tensor")
        nbytes = ws.numel() * ws.element_size()
    _check_bc(d)
    st = _lib().m3_scan_prefill_varlen(ctypes.byref(d), _ptr(cu_seqlens), _ptr(x), _ptr(dt),
                                       _ptr(A), _ptr(lam), _ptr(theta), _ptr(B), _ptr(C),
                                       _ptr(h0), _ptr(x_prev), _ptr(B_prev), _ptr(y), _ptr(hT),
                                       _ptr(ws), nbytes, _stream(stream))
    if st != 0:
        raise M3Error(st, "m3_scan_prefill_varlen")


def m3_decode_step(dims: m3_dims, h, x_t, x_prev, B_t, B_prev, C_t, dt_t, A, lam_t,
                   theta_t, y_t, stream=None) -> None:
    d = dims
    ti, to = _TORCH.get(d.in_dtype), _TORCH.get(d.out_dtype)
    if ti is not None and to is not None:
        Bsz, H, P, N, R = d.batch, d.nheads, d.headdim, d.dstate, d.rank
        G = groups(d)
        _check("h", h, (Bsz, H, P, N), torch.float32)
        _check("x_t", x_t, (Bsz, H, P, R), ti)
        _check("x_prev", x_prev, (Bsz, H, P, R), ti, optional=True)
        _check("B_t", B_t, (Bsz, G, N, R), ti)
        _check("B_prev", B_prev, (Bsz, G, N, R), ti, optional=True)
        _check("C_t", C_t, (Bsz, G, N, R), ti)
        _check("dt_t", dt_t, (Bsz, H), ti)
        _check("A", A, (Bsz, H) if d.flags & M3_A_PER_TOKEN else (H,), torch.float32)
        _check("lam_t", lam_t, (Bsz, H), ti)
        _check("theta_t", theta_t, (Bsz, G, N // 2), ti, optional=_proj(d) is not None)
        if _proj(d) is not None:
            _proj(d).check((Bsz,), G, N, ti)
        _check("y_t", y_t, (Bsz, H, P, R), to)
    _check_bc(d)
    st = _lib().m3_decode_step(ctypes.byref(d), _ptr(h), _ptr(x_t), _ptr(x_prev), _ptr(B_t),
                               _ptr(B_prev), _ptr(C_t), _ptr(dt_t), _ptr(A), _ptr(lam_t),
                               _ptr(theta_t), _ptr(y_t), _stream(stream))
    if st != 0:
        raise M3Error(st, "m3_decode_step")


def m3_decode_tokens(dims: m3_dims, h, x, x_prev, B, B_prev, C, dt, A, lam, theta, y,
                     stream=None) -> None:
    d = dims
    ti, to = _TORCH.get(d.in_dtype), _TORCH.get(d.out_dtype)
    if ti is not None and to is not None:
        Bsz, K, H, P, N, R = d.batch, d.seqlen, d.nheads, d.headdim, d.dstate, d.rank
        G = groups(d)
        _check("h", h, (Bsz, H, P, N), torch.float32)
        _check("x", x, (Bsz, K, H, P, R), ti)
        _check("x_prev", x_prev, (Bsz, H, P, R), ti, optional=True)
        _check("B", B, (Bsz, K, G, N, R), ti)
        _check("B_prev", B_prev, (Bsz, G, N, R), ti, optional=True)
        _check("C", C, (Bsz, K, G, N, R), ti)
        _check("dt", dt, (Bsz, K, H), ti)
        _check("A", A, (Bsz, K, H) if d.flags & M3_A_PER_TOKEN else (H,), torch.float32)
        _check("lam", lam, (Bsz, K, H), ti)
        _check("theta", theta, (Bsz, K, G, N // 2), ti)
        _check("y", y, (Bsz, K, H, P, R), to)
    _check_bc(d)
    st = _lib().m3_decode_tokens(ctypes.byref(d), _ptr(h), _ptr(x), _ptr(x_prev), _ptr(B),
                                 _ptr(B_prev), _ptr(C), _ptr(dt), _ptr(A), _ptr(lam),
                                 _ptr(theta), _ptr(y), _stream(stream))
    if st != 0:
        raise M3Error(st, "m3_decode_tokens")


# ---------------------------------------------------------------------------
# allocation helpers (torch only provides the memory)
def scan_prefill(x, dt, A, lam, theta, B, C, h0=None, x_prev=None, B_prev=None,
                 chunk=0, out_dtype=torch.float32, flags=0, want_hT=True, ws=None,
                 stream=None, bc=None, tp=None):
    """Allocate y (and hT, workspace) and call m3_scan_prefill.  Returns (y, hT).
    B, C and theta may have fewer head slots than x (head groups); with tp
    (a ThetaProj) theta may be None."""
    Bsz, T, H, P, R = x.shape
    G, N = B.shape[2], B.shape[3]
    d = make_dims(Bsz, T, H, P, N, R, chunk, dtype_code(x.dtype), dtype_code(out_dtype), flags,
                  0 if G == H else G, bc, tp)
    y = torch.empty((Bsz, T, H, P, R), dtype=out_dtype, device=x.device)
    hT = torch.empty((Bsz, H, P, N), dtype=torch.float32, device=x.device) if want_hT else None
    if ws is None:
        ws = workspace(d, x.device)
    m3_scan_prefill(d, x, dt, A, lam, theta, B, C, h0, x_prev, B_prev, y, hT, ws, stream)
    return y, hT


def workspace(dims: m3_dims, device, varlen=False) -> torch.Tensor:
    n = (m3_prefill_varlen_workspace_size if varlen else m3_prefill_workspace_size)(dims)
    if n == 0:
        raise M3Error(2, "m3_prefill_workspace_size")
    return torch.empty((n + 15) // 16 * 16, dtype=torch.uint8, device=device)


def scan_prefill_backward(x, dt, A, lam, theta, B, C, dy, h0=None, x_prev=None, B_prev=None,
                          dhT=None, flags=0, chunk=0, stream=None) -> dict:
    """Allocate the fp32 gradients (and workspace) and call
    m3_scan_prefill_backward.  Returns a dict keyed by GRAD_NAMES."""
    Bsz, T, H, P, R = x.shape
    G, N = B.shape[2], B.shape[3]
    d = make_dims(Bsz, T, H, P, N, R, chunk, dtype_code(x.dtype), dtype_code(dy.dtype), flags,
                  0 if G == H else G)
    dev, f32 = x.device, torch.float32
    like = lambda t: None if t is None else torch.empty(t.shape, dtype=f32, device=dev)
    grads = {k: like(v) for k, v in (("x", x), ("dt", dt), ("A", A), ("lam", lam),
                                      ("theta", theta), ("B", B), ("C", C), ("x_prev", x_prev),
                                      ("B_prev", B_prev))}
    grads["h0"] = torch.empty((Bsz, H, P, N), dtype=f32, device=dev) if h0 is not None else None
    n = m3_prefill_backward_workspace_size(d)
    if n == 0:
        raise M3Error(2, "m3_prefill_backward_workspace_size")
    ws = torch.empty((n + 15) // 16 * 16, dtype=torch.uint8, device=dev)
    m3_scan_prefill_backward(d, x, dt, A, lam, theta, B, C, h0, x_prev, B_prev, dy, dhT, grads,
                             ws, stream)
    return grads


def scan_prefill_varlen(cu_seqlens, x, dt, A, lam, theta, B, C, h0=None, x_prev=None,
                        B_prev=None, chunk=0, out_dtype=torch.float32, flags=0, want_hT=True,
                        ws=None, stream=None, bc=None, tp=None):
    """Allocate y (and hT, workspace) and call m3_scan_prefill_varlen on
    sequences packed into x [T, H, P, R].  Returns (y, hT)."""
    T, H, P, R = x.shape
    G, N = B.shape[1], B.shape[2]
    S = cu_seqlens.numel() - 1
    d = make_dims(S, T, H, P, N, R, chunk, dtype_code(x.dtype), dtype_code(out_dtype), flags,
                  0 if G == H else G, bc, tp)
    y = torch.empty((T, H, P, R), dtype=out_dtype, device=x.device)
    hT = torch.empty((S, H, P, N), dtype=torch.float32, device=x.device) if want_hT else None
    if ws is None:
        ws = workspace(d, x.device, varlen=True)
    m3_scan_prefill_varlen(d, cu_seqlens, x, dt, A, lam, theta, B, C, h0, x_prev, B_prev, y,
                           hT, ws, stream)
    return y, hT


def decode_step(h, x_t, B_t, C_t, dt_t, A, lam_t, theta_t, x_prev=None, B_prev=None,
                out_dtype=torch.float32, flags=0, y_t=None, stream=None, bc=None, tp=None):
    """Advance h in place by one token; returns y_t (allocated unless given).
    B_t, C_t and theta_t may have fewer head slots than h (head groups);
    with tp (a ThetaProj) theta_t may be None."""
    Bsz, H, P, N = h.shape
    R = x_t.shape[-1]
    G = B_t.shape[1]
    d = make_dims(Bsz, 1, H, P, N, R, 0, dtype_code(x_t.dtype), dtype_code(out_dtype), flags,
                  0 if G == H else G, bc, tp)
    if y_t is None:
        y_t = torch.empty((Bsz, H, P, R), dtype=out_dtype, device=h.device)
    m3_decode_step(d, h, x_t, x_prev, B_t, B_prev, C_t, dt_t, A, lam_t, theta_t, y_t, stream)
    return y_t


def decode_tokens(h, x, B, C, dt, A, lam, theta, x_prev=None, B_prev=None,
                  out_dtype=torch.float32, flags=0, y=None, stream=None, bc=None):
    """Advance h in place by the K tokens of x ([Bsz, K, H, P, R]); returns y
    ([Bsz, K, H, P, R], allocated unless given)."""
    Bsz, K, H, P, R = x.shape
    N = h.shape[3]
    G = B.shape[2]
    d = make_dims(Bsz, K, H, P, N, R, 0, dtype_code(x.dtype), dtype_code(out_dtype), flags,
                  0 if G == H else G, bc)
    if y is None:
        y = torch.empty((Bsz, K, H, P, R), dtype=out_dtype, device=h.device)
    m3_decode_tokens(d, h, x, x_prev, B, B_prev, C, dt, A, lam, theta, y, stream)
    return y
