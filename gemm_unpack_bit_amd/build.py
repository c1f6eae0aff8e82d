"""Build libqgemv.so in-tree: hipcc for the gfx950 kernels, the host compiler
for the C ABI layer.  Usage: ``python -m gemm_unpack_bit_amd.build``."""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqgemv.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function",
]
CXX_FLAGS = [
    "-O2", "-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__", "-I", f"{ROCM}/include",
    "-I", INCLUDE, "-I", CSRC, "-Wall",
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def sources():
    hip = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    cpp = sorted(f for f in os.listdir(CSRC) if f.endswith(".cpp"))
    return hip, cpp


def build(verbose: bool = False, jobs: int | None = None) -> str:
    hipcc = shutil.which("hipcc") or f"{ROCM}/bin/hipcc"
    cxx = shutil.which("g++") or "c++"
    os.makedirs(BUILD, exist_ok=True)
    hip, cpp = sources()
    jobs = jobs or min(8, os.cpu_count() or 4)
    cmds = []
    objs = []
    for f in hip:
        o = os.path.join(BUILD, f + ".o")
        cmds.append([hipcc, *HIP_FLAGS, "-c", os.path.join(CSRC, f), "-o", o])
        objs.append(o)
    for f in cpp:
        o = os.path.join(BUILD, f + ".o")
        cmds.append([cxx, *CXX_FLAGS, "-c", os.path.join(CSRC, f), "-o", o])
        objs.append(o)
    with cf.ThreadPoolExecutor(jobs) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs,
          f"-L{ROCM}/lib", "-lamdhip64", "-Wl,-soname,libqgemv.so"])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
