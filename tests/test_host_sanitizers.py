"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

tests/host_sanitize.cpp runs the oracle's exported functions on small random
inputs and drives the C ABI's host code (argument checks, workspace sizes,
the weight-gradient split plan) over valid, edge and invalid shapes.  The
oracle and the driver are built with gcc/g++ and both sanitizers; api.cpp is
built by hipcc with the sanitizers on its host pass only; the kernels' objects
are the library's own.  No call reaches a kernel launch."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OBJ = os.path.join(ROOT, "_build", "obj")
OUT = os.path.join(ROOT, "_build", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
KERNEL_OBJS = ["route", "permute", "grouped_gemm", "combine", "norm", "bwd_gemm", "bwd"]


def run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(HIPCC),
                    reason="needs g++ and hipcc")
def test_host_code_is_clean_under_asan_and_ubsan():
    if not all(os.path.exists(os.path.join(OBJ, f"{o}.o")) for o in KERNEL_OBJS):
        from sparse_mixture_experts_51_amd import build
        build.build()
    os.makedirs(OUT, exist_ok=True)
    san = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-g", "-O1"]
    oracle_o = os.path.join(OUT, "oracle.o")
    run(["gcc", "-std=c11", "-mfma", "-ffp-contract=off", *san, "-c",
         os.path.join(ROOT, "oracle", "moe_oracle.c"), "-o", oracle_o])
    api_o = os.path.join(OUT, "api.o")
    run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         "-Xarch_host", "-fno-omit-frame-pointer", "-Wno-unused-command-line-argument",
         "-x", "hip", "-c", os.path.join(ROOT, "sparse_mixture_experts_51_amd", "csrc", "api.cpp"),
         "-o", api_o])
    drv_o = os.path.join(OUT, "driver.o")
    run(["g++", "-std=c++17", *san, "-c", os.path.join(ROOT, "tests", "host_sanitize.cpp"),
         "-o", drv_o])
    exe = os.path.join(OUT, "host_check")
    run(["g++", "-fsanitize=address,undefined", drv_o, oracle_o, api_o,
         *[os.path.join(OBJ, f"{o}.o") for o in KERNEL_OBJS],
         "-L/opt/rocm/lib", "-lamdhip64", "-lm", "-lpthread", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stderr[-5000:]
    assert "clean" in r.stdout
