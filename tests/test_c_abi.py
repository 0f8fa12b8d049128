"""The C ABI used from plain C99 (no GPU needed): tests/c/abi_from_c.c is
compiled with gcc against include/moe_dispatch.h, linked against
libmoe_dispatch.so and run; it calls only paths decided on the host."""
import os
import shutil
import subprocess

import pytest

import combine_topk_idx_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_from_plain_c(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    if not os.path.exists(M.LIB_PATH):
        pytest.fail("libmoe_dispatch.so is not built (python -m combine_topk_idx_amd.build)")
    exe = str(tmp_path / "abi_from_c")
    libdir = os.path.dirname(M.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_from_c.c"),
                    "-L", libdir, "-l:libmoe_dispatch.so", f"-Wl,-rpath,{libdir}", "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "C ABI checks passed" in r.stdout
