"""The C ABI from plain C: tests/c_abi/abi_consumer.c includes only include/gqa.h, is compiled with gcc as
strict C11 and linked against the built libgqa.so, and checks the size queries, every host-side argument
check and the status strings.  No call reaches the GPU (each check fails on the host first)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "gqa_attention_rope_amd")
LIB = os.path.join(PKG, "libgqa.so")
ROCM_LIB = "/opt/rocm/lib"


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_plain_c_consumer(tmp_path):
    if not os.path.exists(LIB):
        pytest.skip("libgqa.so is not built (run __graft_entry__.build())")
    exe = tmp_path / "abi_consumer"
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_abi", "abi_consumer.c"), "-o", str(exe), "-L", PKG, "-lgqa",
           "-Wl,-rpath," + PKG, "-Wl,-rpath-link," + ROCM_LIB, "-Wl,-rpath," + ROCM_LIB]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stdout + build.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    print(run.stdout)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "0 failure(s)" in run.stdout
