"""The C ABI layer (combine_moe_layout_02_amd/csrc/moe_api.cpp) compiled for the host with g++ and
the address and undefined-behaviour sanitizers, linked against stand-in launchers that only count
calls (tests/c_abi/abi_stubs.cpp), and driven by tests/c_abi/abi_asan.cpp: size arithmetic at the
limits and at hostile int64 arguments, rejected calls, and which launchers valid calls reach.
Runs on the CPU; no GPU code is built or run."""

import os
import shutil
import subprocess

import pytest

from conftest import ROOT

C_ABI = os.path.join(ROOT, "tests", "c_abi")
CSRC = os.path.join(ROOT, "combine_moe_layout_02_amd", "csrc")


def test_abi_layer_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"):
        pytest.skip("needs g++ and the HIP headers")
    exe = tmp_path / "abi_asan"
    cmd = [gxx, "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", f"-I{C_ABI}",
           os.path.join(CSRC, "moe_api.cpp"), os.path.join(C_ABI, "abi_stubs.cpp"),
           os.path.join(C_ABI, "abi_asan.cpp"), "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=60)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "abi_asan ok" in run.stdout
