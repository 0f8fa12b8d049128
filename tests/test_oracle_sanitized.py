"""The oracle's C under AddressSanitizer and UBSan (host only).

tests/c/oracle_sanitize.c drives every exported oracle function over small
seeded inputs (both layouts, every activation format, invalid and unrouted
ids, masked overflow, zero tokens, one and four threads).  It is built with
oracle/oracle.c by gcc with -fsanitize=address,undefined and
-fno-sanitize-recover=all, so any out-of-bounds access, leak or undefined
operation ends the run with a nonzero status.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "c", "oracle_sanitize.c")
ORACLE = os.path.join(ROOT, "oracle", "oracle.c")


def test_oracle_runs_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    flags = ["-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer", "-fopenmp", "-ffp-contract=off", "-Wall", "-Wextra", "-Werror"]
    build = subprocess.run(["gcc", *flags, DRIVER, ORACLE, "-lm", "-o", exe], capture_output=True, text=True)
    if build.returncode != 0 and "cannot find" in build.stderr and "asan" in build.stderr:
        pytest.skip("gcc has no sanitizer runtime here")
    assert build.returncode == 0, build.stderr
    env = dict(os.environ)
    # a preloaded library ahead of the ASan runtime is allowed; leaks are reported
    env["ASAN_OPTIONS"] = "detect_leaks=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "oracle ran clean" in run.stdout
