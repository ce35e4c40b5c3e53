"""Build libmoe.so (the HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Run as ``python combine_moe_layout_02_amd/build.py`` (a path, so that the package, which loads
libmoe.so at import, is not imported first) or through ``__graft_entry__.build()``. Always
recompiles. The library lands next to this file, where the Python binding loads it.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmoe.so")
ARCH = "gfx950"

SOURCES = ["layout.hip", "layout_small.hip", "pack.hip", "pack_planned.hip", "combine.hip", "unpack.hip",
           "probe.hip", "noalloc.hip", "moe_api.cpp"]

# -ffp-contract=off: combine rounds every product and sum to fp32 on its own (no fused multiply-add).
# -packed-fp32-ops off: scalar fp32 only; no packed fp32 instructions are generated.
FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libmoe.so")
    return path


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return res


def build(verbose=False, extra_flags=()):
    cc = hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [cc, "-x", "hip", *FLAGS, *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        _run(cmd)
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    _run(cmd)
    os.replace(tmp, LIB)
    return LIB


def build_abi_harness(verbose=False):
    """The native test programs the GPU tests run, each landing next to its source:
    tests/c_abi/abi_gpu.cpp, a C++ consumer of the C ABI linked against libmoe.so, and
    tests/c_abi/quant_gpu.cpp, which runs the pack's quantisation helpers (csrc/pack_rows.h) over
    every fp32 code boundary and every bf16 quotient, compiled with the library's flags."""
    c_abi = os.path.join(ROOT, "tests", "c_abi")
    abi = os.path.join(c_abi, "abi_gpu")
    cmds = [[hipcc(), "-x", "hip", "-O2", "-std=c++17", f"--offload-arch={ARCH}", f"-I{INCLUDE}",
             os.path.join(c_abi, "abi_gpu.cpp"), "-o", abi, f"-L{PKG}", "-lmoe", f"-Wl,-rpath,{PKG}"]]
    quant = os.path.join(c_abi, "quant_gpu")
    flags = [f for f in FLAGS if f not in ("-fPIC",)]
    cmds.append([hipcc(), "-x", "hip", *flags, os.path.join(c_abi, "quant_gpu.cpp"), "-o", quant])
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        _run(cmd)
    return [abi, quant]


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_abi_harness(verbose="-v" in sys.argv))
