"""The C ABI from a C program: tests/c/abi_check.c, compiled as C11 with
gcc (warnings as errors, -pedantic) against include/msa.h and linked to the
built libmsa.so, takes the address of every entry point and runs the
host-side checks that need no GPU."""
import os
import shutil
import subprocess

import pytest

from block_sparse_attention_kv_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c_client_compiles_links_and_runs(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    lib = os.path.abspath(_lib.LIB_PATH)
    assert os.path.exists(lib), "libmsa.so is not built"
    libdir = os.path.dirname(lib)
    exe = str(tmp_path / "abi_check")
    cmd = [gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_check.c"), "-L", libdir, "-lmsa", "-Wl,-rpath," + libdir, "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert run.stdout.startswith("ok "), run.stdout
