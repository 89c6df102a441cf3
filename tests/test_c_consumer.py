"""The C ABI from plain C: tests/c/abi_consumer.c is compiled as C99 with
-Wall -Werror against include/mi_attn.h, linked against the built
libmi_attn.so and run.  It needs no GPU (only library queries and argument
errors reported before any HIP call)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "exact_attention_61_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_consumer(tmp_path):
    assert os.path.exists(os.path.join(LIBDIR, "libmi_attn.so")), "library not built"
    exe = str(tmp_path / "abi_consumer")
    build = subprocess.run(
        ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
         os.path.join(ROOT, "tests", "c", "abi_consumer.c"), "-o", exe, "-L", LIBDIR,
         "-lmi_attn", "-Wl,-rpath," + LIBDIR, "-lm"],
        capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "all checks passed" in run.stdout
