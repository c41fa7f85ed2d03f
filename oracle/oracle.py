"""Python face of the fp64 CPU oracle -- TEST INFRASTRUCTURE ONLY.

The oracle is the plain sequential Mamba-3 core recurrence written in C
(``m3_oracle.c``; see its header for what it computes and the pages it
follows).  This module compiles it with gcc and calls it through ctypes on
numpy float64 arrays.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import it; the HIP library never does.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "m3_oracle.c")
_OUT_DIR = os.path.join(_HERE, "_build")
_LIB = os.path.join(_OUT_DIR, "libm3oracle.so")

THETA_IS_ANGLE = 1
A_PER_TOKEN = 2


class _Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("nheads", ctypes.c_int64), ("headdim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("rank", ctypes.c_int64),
                ("flags", ctypes.c_uint32)]


def build(src: str = _SRC, out: str = _LIB, extra: tuple = ()) -> str:
    """Compile the oracle (plain -O2, no fast-math, OpenMP over (b,h))."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-Wextra", *extra, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


_lib_cache: dict = {}


def load(path: str = _LIB) -> ctypes.CDLL:
    if path in _lib_cache:
        return _lib_cache[path]
    if not os.path.exists(path) or (
            path == _LIB and os.path.getmtime(path) < os.path.getmtime(_SRC)):
        build(out=path)
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.m3ref_scan.restype = ctypes.c_int
    lib.m3ref_scan.argtypes = [ctypes.POINTER(_Dims)] + [dp] * 12 + [ctypes.c_int]
    lib.m3ref_decode_step.restype = ctypes.c_int
    lib.m3ref_decode_step.argtypes = [ctypes.POINTER(_Dims)] + [dp] * 11 + [ctypes.c_int]
    lib.m3ref_scan_backward.restype = ctypes.c_int
    lib.m3ref_scan_backward.argtypes = [ctypes.POINTER(_Dims)] + [dp] * 22 + [ctypes.c_int]
    lib.m3ref_bc_prep.restype = ctypes.c_int
    lib.m3ref_bc_prep.argtypes = [ctypes.c_int64] * 5 + [dp] * 3 + [ctypes.c_double,
                                                                    ctypes.c_int, dp]
    lib.m3ref_theta_proj.restype = ctypes.c_int
    lib.m3ref_theta_proj.argtypes = [ctypes.c_int64] * 4 + [dp] * 3
    lib.m3ref_max_threads.restype = ctypes.c_int
    _lib_cache[path] = lib
    return lib


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


@dataclass
class ScanResult:
    y: np.ndarray
    hT: np.ndarray


def scan(x, dt, A, lam, theta, B, C, h0=None, x_prev=None, B_prev=None,
         flags: int = 0, nthreads: int = 0, lib_path: str = _LIB) -> ScanResult:
    """Sequential fp64 scan.  Shapes: x [Bsz,T,H,P,R], B/C [Bsz,T,H,N,R],
    dt/lam [Bsz,T,H], theta [Bsz,T,H,N/2], A [H] (or [Bsz,T,H] with
    A_PER_TOKEN), h0 [Bsz,H,P,N], x_prev [Bsz,H,P,R], B_prev [Bsz,H,N,R]."""
    lib = load(lib_path)
    x, dt, A, lam, theta, B, C = map(_f64, (x, dt, A, lam, theta, B, C))
    h0, x_prev, B_prev = map(_f64, (h0, x_prev, B_prev))
    Bsz, T, H, P, R = x.shape
    N = B.shape[3]
    d = _Dims(Bsz, T, H, P, N, R, flags)
    y = np.zeros((Bsz, T, H, P, R), np.float64)
    hT = np.zeros((Bsz, H, P, N), np.float64)
    rc = lib.m3ref_scan(ctypes.byref(d), _ptr(x), _ptr(dt), _ptr(A), _ptr(lam),
                        _ptr(theta), _ptr(B), _ptr(C), _ptr(h0), _ptr(x_prev),
                        _ptr(B_prev), _ptr(y), _ptr(hT), int(nthreads))
    if rc:
        raise ValueError("m3ref_scan rejected its arguments (code %d)" % rc)
    return ScanResult(y, hT)


def decode_step(h, x_t, x_prev, B_t, B_prev, C_t, dt_t, A, lam_t, theta_t,
                flags: int = 0, nthreads: int = 0, lib_path: str = _LIB):
    """One token: returns (y_t [Bsz,H,P,R], h_new [Bsz,H,P,N]); h is not
    modified.  x_prev/B_prev may be None (zero)."""
    lib = load(lib_path)
    h = np.array(h, dtype=np.float64, copy=True, order="C")
    x_t, x_prev, B_t, B_prev, C_t = map(_f64, (x_t, x_prev, B_t, B_prev, C_t))
    dt_t, A, lam_t, theta_t = map(_f64, (dt_t, A, lam_t, theta_t))
    Bsz, H, P, R = x_t.shape
    N = B_t.shape[2]
    d = _Dims(Bsz, 1, H, P, N, R, flags)
    y = np.zeros((Bsz, H, P, R), np.float64)
    rc = lib.m3ref_decode_step(ctypes.byref(d), _ptr(h), _ptr(x_t), _ptr(x_prev),
                               _ptr(B_t), _ptr(B_prev), _ptr(C_t), _ptr(dt_t),
                               _ptr(A), _ptr(lam_t), _ptr(theta_t), _ptr(y),
                               int(nthreads))
    if rc:
        raise ValueError("m3ref_decode_step rejected its arguments (code %d)" % rc)
    return y, h


GRAD_NAMES = ("x", "dt", "A", "lam", "theta", "B", "C", "h0", "x_prev", "B_prev")


def scan_backward(x, dt, A, lam, theta, B, C, h0=None, x_prev=None, B_prev=None, dy=None,
                  dhT=None, flags: int = 0, nthreads: int = 0, lib_path: str = _LIB) -> dict:
    """Gradients of L = <y, dy> + <hT, dhT> with respect to every input of
    scan() (same layouts; dA is [H] unless A_PER_TOKEN).  Returns a dict keyed
    by GRAD_NAMES; the entries of h0 / x_prev / B_prev are None when those
    inputs are None."""
    lib = load(lib_path)
    x, dt, A, lam, theta, B, C = map(_f64, (x, dt, A, lam, theta, B, C))
    h0, x_prev, B_prev, dy, dhT = map(_f64, (h0, x_prev, B_prev, dy, dhT))
    Bsz, T, H, P, R = x.shape
    N = B.shape[3]
    d = _Dims(Bsz, T, H, P, N, R, flags)
    prev = x_prev is not None and B_prev is not None
    g = {k: np.zeros_like(v) for k, v in (("x", x), ("dt", dt), ("A", A), ("lam", lam),
                                           ("theta", theta), ("B", B), ("C", C))}
    g["h0"] = np.zeros((Bsz, H, P, N)) if h0 is not None else None
    g["x_prev"] = np.zeros_like(x_prev) if prev else None
    g["B_prev"] = np.zeros_like(B_prev) if prev else None
    dh0 = g["h0"] if g["h0"] is not None else np.zeros((Bsz, H, P, N))
    rc = lib.m3ref_scan_backward(ctypes.byref(d), _ptr(x), _ptr(dt), _ptr(A), _ptr(lam),
                                 _ptr(theta), _ptr(B), _ptr(C), _ptr(h0), _ptr(x_prev),
                                 _ptr(B_prev), _ptr(dy), _ptr(dhT), _ptr(g["x"]), _ptr(g["dt"]),
                                 _ptr(g["A"]), _ptr(g["lam"]), _ptr(g["theta"]), _ptr(g["B"]),
                                 _ptr(g["C"]), _ptr(dh0), _ptr(g["x_prev"]), _ptr(g["B_prev"]),
                                 int(nthreads))
    if rc:
        raise ValueError("m3ref_scan_backward rejected its arguments (code %d)" % rc)
    return g


def bc_prep(v, nheads, weight=None, bias=None, eps=1e-6, rms=True, lib_path: str = _LIB):
    """B or C as the recurrence sees them after the section-2 preparation:
    v [..., G, N, R] (one slot per head group) -> [..., H, N, R], each head
    normalised over N per rank column, scaled by weight [N] and offset by its
    own bias [H, N, R] (see m3ref_bc_prep)."""
    lib = load(lib_path)
    v = _f64(v)
    *lead, G, N, R = v.shape
    rows = int(np.prod(lead)) if lead else 1
    out = np.zeros(tuple(lead) + (nheads, N, R), np.float64)
    rc = lib.m3ref_bc_prep(rows, G, nheads, N, R, _ptr(v), _ptr(_f64(weight)),
                           _ptr(_f64(bias)), float(eps), int(bool(rms)), _ptr(out))
    if rc:
        raise ValueError("m3ref_bc_prep rejected its arguments (code %d)" % rc)
    return out


def theta_proj(u, W, lib_path: str = _LIB):
    """Angles from the projection: u [..., D], W [G, K, D] -> [..., G, K]."""
    lib = load(lib_path)
    u, W = _f64(u), _f64(W)
    lead = u.shape[:-1]
    D = u.shape[-1]
    G, K, D2 = W.shape
    if D2 != D:
        raise ValueError("W and u disagree on the projection width")
    rows = int(np.prod(lead)) if lead else 1
    out = np.zeros(tuple(lead) + (G, K), np.float64)
    rc = lib.m3ref_theta_proj(rows, G, K, D, _ptr(u), _ptr(W), _ptr(out))
    if rc:
        raise ValueError("m3ref_theta_proj rejected its arguments (code %d)" % rc)
    return out


def max_threads(lib_path: str = _LIB) -> int:
    return int(load(lib_path).m3ref_max_threads())
