"""The oracle and the host side of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

Each test builds a small driver (tests/san/) together with the code under
test, instrumented, into an executable of its own in a temporary folder, and
runs it: the driver calls every entry point over edge-case shapes (one block,
k = 0, k = K, empty and ragged shapes, padded rows, the most segments and
groups, every argument error) and exits non-zero on a failed check or on any
sanitizer report, leaks included.  Only host code is instrumented: the
library's device code is compiled as usual and never runs here.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "san")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-6000:]}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    if not os.path.exists(subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                                         text=True).stdout.strip()):
        pytest.skip("gcc has no AddressSanitizer runtime here")
    exe = str(tmp_path / "oracle_san")
    run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-omit-frame-pointer",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all", os.path.join(SAN, "oracle_san.c"),
         os.path.join(ROOT, "oracle", "oracle.c"), "-o", exe, "-lm"])
    r = run([exe], env=ENV, timeout=300)
    assert "oracle sanitizer run: ok" in r.stdout


def test_abi_host_code_under_asan_ubsan(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)):
        pytest.skip("no HIP toolchain here")
    csrc = os.path.join(ROOT, "fp4_gemm_sparse_amd", "csrc")
    objs = []
    procs = []
    for src in ("api", "quant", "gemm", "fused", "tim", "probe"):
        obj = str(tmp_path / f"{src}.o")
        objs.append(obj)
        # sanitizers on the host pass only; the device code is built as usual
        procs.append(subprocess.Popen(
            [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-ffp-contract=off",
             "-fno-omit-frame-pointer", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-c", os.path.join(csrc, src + ".hip"), "-o", obj],
            stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    for p, src in zip(procs, ("api", "quant", "gemm", "fused", "tim", "probe")):
        out, err = p.communicate(timeout=600)
        assert p.returncode == 0, f"{src}.hip:\n{err[-4000:]}"
    drv = str(tmp_path / "abi_san.o")
    run([CLANGXX, "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-c", os.path.join(SAN, "abi_san.cpp"), "-o", drv])
    exe = str(tmp_path / "abi_san")
    run([CLANGXX, "-fsanitize=address,undefined", drv, *objs, "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib",
         "-lamdhip64", "-o", exe])
    r = run([exe], env=ENV, timeout=300)
    assert "ABI sanitizer run: ok" in r.stdout
