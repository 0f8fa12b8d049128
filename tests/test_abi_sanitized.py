"""The library's host code under AddressSanitizer and UBSan.

The library is built from its sources with the sanitizers on the host side
only (each -fsanitize flag behind -Xarch_host; the device code is the
ordinary gfx950 build), and tests/c/abi_from_c.c -- size queries, config
validation, and every entry point's argument errors, which return before
anything reaches a GPU -- is built with clang's sanitizers against it and run.
No call launches a kernel, so this runs without a GPU.
"""
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def test_host_code_runs_clean_under_asan_and_ubsan(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("hipcc or ROCm's clang not available")
    lib = str(tmp_path / "libmoe_dispatch_sanitized.so")
    srcs = sorted(glob.glob(os.path.join(ROOT, "combine_topk_idx_amd", "csrc", "*.hip")))
    build = subprocess.run(
        [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_SANITIZE,
         "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "combine_topk_idx_amd", "csrc"),
         "-o", lib, *srcs], capture_output=True, text=True, timeout=600)
    assert build.returncode == 0, build.stderr[-4000:]
    exe = str(tmp_path / "abi_from_c_sanitized")
    link = subprocess.run(
        [CLANG, "-std=c99", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_from_c.c"), lib,
         f"-Wl,-rpath,{tmp_path}", "-o", exe], capture_output=True, text=True, timeout=300)
    assert link.returncode == 0, link.stderr[-4000:]
    env = dict(os.environ)
    # the HIP runtime's own allocations are not this library's: no leak report;
    # a preloaded library ahead of the ASan runtime is allowed
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "C ABI checks passed" in run.stdout
