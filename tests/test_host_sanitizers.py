"""Host-side AddressSanitizer / UndefinedBehaviorSanitizer runs (no GPU).

* The fp64 oracle is rebuilt with gcc's ASan + UBSan and every pin of
  tests/oracle_pins.py runs against that build, in a child process that
  preloads gcc's ASan runtime.  A copy of the oracle with a planted
  one-past-the-end read must make that run fail, so the harness is known to
  catch what it is for.
* The C ABI layer (api.cpp: argument checks, workspace sizing) is rebuilt
  with clang's ASan + UBSan for the host side only, linked with the kernel
  objects of the normal build, and tests/test_abi.py (every error path of
  every entry point; none of them launches a kernel) runs against it in a
  child process that preloads clang's ASan runtime.

Leak checking is off: the HIP runtime keeps allocations until exit."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

from oracle import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "linear_recurrent_sequence_mamba_amd")
SAN_ENV = dict(ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
PINS = """
import sys
sys.path.insert(0, {root!r})
from tests import oracle_pins as p
for c in p.ALL_CHECKS:
    c({lib!r})
print("PINS_OK", flush=True)
"""


def _run(code, preload, timeout=300):
    env = dict(os.environ, LD_PRELOAD=preload, **SAN_ENV)
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=timeout)


def _gcc_asan():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc's ASan runtime is not installed")
    return path


def _build_oracle(src, out):
    oracle.build(src=src, out=out, extra=("-O1", "-g", "-fno-omit-frame-pointer",
                                          "-fsanitize=address,undefined",
                                          "-fno-sanitize-recover=undefined", "-w"))


def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    _build_oracle(oracle._SRC, lib)
    r = _run(PINS.format(root=ROOT, lib=lib), _gcc_asan())
    assert r.returncode == 0 and "PINS_OK" in r.stdout, r.stderr[-3000:]


def test_oracle_sanitizer_catches_a_planted_overflow(tmp_path):
    """The same run on an oracle that reads one angle past each token's row
    (past the end of the array on the last token) must fail."""
    src = open(oracle._SRC).read()
    old = "const double cs = cos(phi), sn = sin(phi);"
    assert old in src
    bad = src.replace(old, "const double cs = cos(phi), sn = sin(phi) + 0.0 * theta[k + 1];")
    msrc = tmp_path / "m3_oracle_oob.c"
    msrc.write_text(bad)
    lib = str(tmp_path / "liboracle_oob.so")
    _build_oracle(str(msrc), lib)
    r = _run(PINS.format(root=ROOT, lib=lib), _gcc_asan())
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, r.stderr[-2000:]


def _hipcc():
    h = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
    if not os.path.exists(h):
        pytest.skip("hipcc is not installed")
    return h


def _clang_asan(hipcc):
    rt = glob.glob(os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "llvm", "lib",
                                "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so"))
    rt += glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not rt:
        pytest.skip("clang's ASan runtime is not installed")
    return os.path.realpath(rt[0])


def test_abi_error_paths_under_asan_ubsan(tmp_path):
    from linear_recurrent_sequence_mamba_amd import build as libbuild
    hipcc = _hipcc()
    kernels = [os.path.join(libbuild.OUT_DIR, s + ".o") for s in libbuild.SOURCES
               if s.endswith(".hip")]
    if not all(os.path.exists(k) for k in kernels):
        libbuild.build()
    # host-only instrumentation: each sanitizer flag goes to the host pass
    host = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
            "-fno-omit-frame-pointer"]
    obj = str(tmp_path / "api_san.o")
    cmd = [hipcc, "-x", "hip", f"--offload-arch={libbuild.ARCH}", "-O1", "-g", "-fPIC",
           "-std=c++17", *host, "-c", os.path.join(libbuild.CSRC, "api.cpp"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    lib = str(tmp_path / "libm3ssm_san.so")
    cmd = [hipcc, f"--offload-arch={libbuild.ARCH}", "-shared", "-fPIC", "-shared-libsan", *host,
           obj, *kernels, "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    code = f"""
import sys
sys.path.insert(0, {ROOT!r})
from linear_recurrent_sequence_mamba_amd import binding as m3
m3.LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main([{os.path.join(ROOT, 'tests', 'test_abi.py')!r}, "-q", "-s", "-p",
                      "no:cacheprovider", "-k", "not binding_rejects"]))
"""
    r = _run(code, _clang_asan(hipcc))
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-3000:])
