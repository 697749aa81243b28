"""The C ABI from plain C (CPU only): tests/c/abi_check.c includes every header under
include/ as C11 (gcc, -Wall -Wextra -Werror -pedantic), links libkvbt.so and checks the
host-side entry points -- launch policy, status strings, version and argument
validation -- with no GPU call."""
import os
import shutil
import subprocess

import pytest

import kv_block_top_amd as kvbt

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_headers_compile_as_c_and_host_calls_behave(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    kvbt.lib()                       # raises if the library is not built
    lib_dir = os.path.dirname(kvbt.library_path())
    exe = str(tmp_path / "abi_check")
    cmd = [gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "c", "abi_check.c"),
           "-L", lib_dir, "-lkvbt", "-Wl,-rpath," + lib_dir, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "C ABI checks passed" in r.stdout


def test_launch_divisor_matches_exact_division(tmp_path):
    """The multiply-and-shift division the kernels use for the heads per row and the
    decode query length (kv_block_top_amd/csrc/kvbt_divide.h), against the exact
    quotient on the host."""
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "divisor_check")
    cmd = [gxx, "-std=c++17", "-O2", "-Wall", "-Wextra", "-Werror",
           "-I", os.path.join(ROOT, "kv_block_top_amd", "csrc"),
           os.path.join(HERE, "c", "divisor_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "divisor checks passed" in r.stdout
