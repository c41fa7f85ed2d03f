"""Build libm3ssm.so in-tree with hipcc for gfx950.

    python -m linear_recurrent_sequence_mamba_amd.build

Each translation unit is compiled on its own (in parallel) and linked into
``linear_recurrent_sequence_mamba_amd/libm3ssm.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libm3ssm.so")
SOURCES = ["api.cpp", "backward.hip", "backward_mma.hip", "decode.hip", "decode_tokens.hip",
           "prefill.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          # keep the compiler from emitting packed fp32 VALU instructions
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument"]


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if r.stderr.strip():
        sys.stderr.write(_filter_warnings(r.stderr))
    return obj


def _filter_warnings(text: str) -> str:
    # hipcc's host pass does not know the packed-fp32 feature; that note is harmless
    keep = [ln for ln in text.splitlines(True) if "packed-fp32-ops" not in ln
            and "not a recognized feature" not in ln]
    return "".join(keep)


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
