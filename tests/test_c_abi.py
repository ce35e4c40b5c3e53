"""The boundary from C: a plain C program (tests/c_abi/abi_host.c) includes include/moe.h, links
libmoe.so and calls the host-only entry points and the host-side validation of the device entry
points. Needs no GPU: nothing reaches a kernel launch."""

import os
import shutil
import subprocess

import pytest

import combine_moe_layout_02_amd as moe
from conftest import ROOT

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("gcc") is None or not os.path.isdir(os.path.join(ROCM, "include", "hip")),
                    reason="needs gcc and the HIP headers")
def test_c_program_uses_the_abi(tmp_path):
    src = os.path.join(ROOT, "tests", "c_abi", "abi_host.c")
    exe = tmp_path / "abi_host"
    libdir = os.path.dirname(moe._LIB_PATH)
    cmd = ["gcc", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{os.path.join(ROCM, 'include')}", src, "-o", str(exe),
           f"-L{libdir}", "-lmoe", f"-Wl,-rpath,{libdir}"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "0 failure(s)" in run.stdout
