"""Undefined behaviour and memory errors in the host code, caught by AddressSanitizer and
UndefinedBehaviorSanitizer builds (CPU only):
  * the task-order checker, built from the rule header the persistent kernels include;
  * the oracle's C sweep, run on ragged random problems (its codes must equal those of
    the ordinary build);
  * the host side of the library (argument checks, workspace sizing, error paths), with
    the ABI tests run against a build whose host code is instrumented.
Each sanitizer build stops at its first report (-fno-sanitize-recover), so a clean exit is
the pass condition."""
import hashlib
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

import oracle
from synthetic import make_random

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "two_sided_adaptive_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV_NO_LEAKS = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0",
                "UBSAN_OPTIONS": "print_stacktrace=1"}


def _run(cmd, env=None, timeout=600):
    full = dict(os.environ)
    full.update(env or {})
    res = subprocess.run(cmd, capture_output=True, text=True, env=full, timeout=timeout,
                         cwd=ROOT)
    out = res.stdout + res.stderr
    assert res.returncode == 0, f"{' '.join(cmd)} failed ({res.returncode}):\n{out[-4000:]}"
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    return out


def test_schedule_checker_clean(tmp_path):
    exe = str(tmp_path / "schedule_check_san")
    _run(["g++", "-O1", "-g", "-std=c++17"] + SAN +
         ["-I", CSRC, os.path.join(ROOT, "tests", "native", "schedule_check.cpp"), "-o", exe])
    for args in (["factor", "64", "64"], ["factor", "224", "64"], ["factor", "10", "17"],
                 ["factor", "2", "3"], ["factor", "1", "1"], ["sweep", "64", "64"],
                 ["sweep", "224", "64"], ["sweep", "5", "9"], ["sweep", "1", "1"],
                 ["run", "21", "6", "3", "2", "1", "1", "2", "1", "2"]):
        _run([exe] + args, env=ENV_NO_LEAKS)


SHAPES = [(37, 29, 3), (64, 65, 4), (1, 7, 2), (130, 3, 8), (17, 128, 5)]

_CHILD = """
import hashlib, sys
sys.path.insert(0, {root!r})
import numpy as np
import oracle.gptq2d as og
og._LIB = {lib!r}
og._lib_handle = None
from synthetic import make_random
for m, n, bits in {shapes!r}:
    wl = make_random(m, n, bits, seed=m * 131 + n)
    z = og.quantize(wl.W, wl.A, wl.B, wl.scales, bits)["Z"]
    print(m, n, hashlib.sha256(np.ascontiguousarray(z, dtype=np.int32).tobytes()).hexdigest())
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_oracle_c_sweep_clean(tmp_path):
    lib = str(tmp_path / "nested_sweep_san.so")
    _run(["gcc", "-O1", "-g", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
          "-shared"] + SAN + ["-o", lib, os.path.join(ROOT, "oracle", "nested_sweep.c"), "-lm"])
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    env = dict(ENV_NO_LEAKS, LD_PRELOAD=asan)
    out = _run([sys.executable, "-c", _CHILD.format(root=ROOT, lib=lib, shapes=SHAPES)],
               env=env)
    got = dict((tuple(map(int, line.split()[:2])), line.split()[2])
               for line in out.splitlines() if line and line[0].isdigit())
    for m, n, bits in SHAPES:
        wl = make_random(m, n, bits, seed=m * 131 + n)
        z = oracle.quantize(wl.W, wl.A, wl.B, wl.scales, bits)["Z"]
        want = hashlib.sha256(np.ascontiguousarray(z, dtype=np.int32).tobytes()).hexdigest()
        assert got[(m, n)] == want, (m, n)


def _clang_asan_runtime():
    base = "/opt/rocm/llvm/lib/clang"
    if not os.path.isdir(base):
        return None
    for ver in sorted(os.listdir(base), reverse=True):
        p = os.path.join(base, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    return None


@pytest.mark.skipif(_clang_asan_runtime() is None or not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc or its AddressSanitizer runtime is missing")
def test_host_library_clean(tmp_path):
    from two_sided_adaptive_amd import build
    lib = str(tmp_path / "libgptq2d_san.so")
    host_san = []
    for flag in SAN:  # host code only: the device code is built as usual
        host_san += ["-Xarch_host", flag]
    _run([build.HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={build.ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + host_san +
         ["-I", os.path.join(ROOT, "include"), "-o", lib] +
         [os.path.join(CSRC, s) for s in build.SOURCES], timeout=900)
    env = dict(ENV_NO_LEAKS, LD_PRELOAD=_clang_asan_runtime(), GPTQ2D_LIB=lib)
    _run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
          os.path.join(ROOT, "tests", "test_abi.py")], env=env)
