"""The C-ABI from plain C: tests/c/abi_consumer.c is compiled with gcc against
include/dflash.h, linked with the built libdflash.so and run (host-side calls
only, no device needed)."""

import os
import shutil
import subprocess

import pytest

from block_diffusion_drafting_ctx_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_plain_c_consumer(tmp_path):
    if not os.path.exists(_abi.LIB_PATH):
        pytest.fail(f"{_abi.LIB_PATH} is missing: build the library first")
    libdir = os.path.dirname(_abi.LIB_PATH)
    exe = str(tmp_path / "abi_consumer")
    cc = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                         os.path.join(ROOT, "tests", "c", "abi_consumer.c"), "-L", libdir, "-ldflash",
                         f"-Wl,-rpath,{libdir}", "-o", exe], capture_output=True, text=True)
    assert cc.returncode == 0, cc.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "0 failed checks" in run.stdout
