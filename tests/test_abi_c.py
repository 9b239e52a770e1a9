"""The C ABI from plain C: tests/c/abi_host_checks.c is compiled with gcc
against include/tbq4.h, linked against the built libtbq4.so and run (host-side
checks only: no GPU needed, no kernel launched)."""

import os
import shutil
import subprocess

import pytest

from long_context_attention_tbq4_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c_program_links_and_passes_host_checks(tmp_path):
    lib = _lib.LIB_PATH
    exe = tmp_path / "abi_host_checks"
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_host_checks.c"), "-o", str(exe),
                    lib, "-Wl,-rpath," + os.path.dirname(lib)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all host-side ABI checks passed" in r.stdout
