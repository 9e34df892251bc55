"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the library's sources with the host side instrumented (the device code
is compiled as usual and never runs here) and links them into
tests/host_sanitize/abi_driver.cpp, which calls every entry point with invalid
and extreme arguments that the host checks must reject, and with zero-sized
calls that return before any launch; no GPU is needed. Any out-of-bounds
access or undefined operation in that host code (a size product that
overflows int64, a shift past the width, ...) aborts the driver. The build is
cached by a hash of its inputs, so only the first run after a source change
compiles (about a minute and a half).
"""
import hashlib
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_quantized_matmul_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
DRIVER = os.path.join(ROOT, "tests", "host_sanitize", "abi_driver.cpp")
BUILD = os.path.join(ROOT, "tests", "host_sanitize", "_build")
SOURCES = ["qmm_api", "dequant", "gemv", "gemv_stream", "gemm", "route"]
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SAN, "-I", INCLUDE, "-I", CSRC]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


def _inputs_hash():
    h = hashlib.sha256(" ".join(FLAGS).encode())
    names = sorted(os.listdir(CSRC)) + ["../../include/qmm.h"]
    for name in names:
        path = os.path.normpath(os.path.join(CSRC, name))
        if os.path.isfile(path):
            h.update(name.encode())
            h.update(open(path, "rb").read())
    h.update(open(DRIVER, "rb").read())
    return h.hexdigest()


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)} failed:\n{res.stdout[-4000:]}\n{res.stderr[-4000:]}")


def _build(hipcc):
    os.makedirs(BUILD, exist_ok=True)
    stamp = os.path.join(BUILD, "inputs.sha256")
    exe = os.path.join(BUILD, "abi_driver")
    digest = _inputs_hash()
    if os.path.exists(exe) and os.path.exists(stamp) and open(stamp).read() == digest:
        return exe
    objs = [os.path.join(BUILD, s + ".o") for s in SOURCES]
    jobs = [[hipcc, *FLAGS, "-c", os.path.join(CSRC, s + ".hip"), "-o", o] for s, o in zip(SOURCES, objs)]
    drv = os.path.join(BUILD, "abi_driver.o")
    jobs.append([hipcc, *FLAGS, "-x", "c++", "-c", DRIVER, "-o", drv])
    with ThreadPoolExecutor(min(len(jobs), os.cpu_count() or 1)) as ex:
        list(ex.map(_run, jobs))
    _run([hipcc, "--offload-arch=gfx950", *SAN, drv, *objs, "-o", exe])
    with open(stamp, "w") as f:
        f.write(digest)
    return exe


def test_abi_checks_under_host_sanitizers():
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not found")
    exe = _build(hipcc)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, f"driver failed ({res.returncode}):\n{res.stdout}\n{res.stderr[-6000:]}"
    assert "abi checks ok" in res.stdout
