"""Build libmm.so in-tree with hipcc for gfx950.

``python -m onnx_broadcast_matmul_amd.build`` (or ``build()``) always
recompiles every source; objects go to ``_build/`` next to this file and the
library to ``onnx_broadcast_matmul_amd/libmm.so``.
"""
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmm.so")

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

COMMON = ["-std=c++17", "-fPIC", "-O3", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall"]
# Packed FP32 instructions are kept out of every device build.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def sources():
    hip = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    cpp = sorted(f for f in os.listdir(CSRC) if f.endswith(".cpp"))
    return hip, cpp


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hip, cpp = sources()
    cmds = []
    objs = []
    for f in hip:
        o = os.path.join(BUILD, f + ".o")
        objs.append(o)
        cmds.append([HIPCC, *DEVICE, *COMMON, "-c", os.path.join(CSRC, f), "-o", o])
    for f in cpp:
        o = os.path.join(BUILD, f + ".o")
        objs.append(o)
        cmds.append([HIPCC, "-x", "c++", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", *COMMON, "-c", os.path.join(CSRC, f), "-o", o])
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    # The LDS-load asm writes M0 behind the compiler's back: refuse a build
    # in which the compiler uses M0 in the same kernels.
    from . import m0check

    m0check.check_objects([o for o in objs if o.endswith(".hip.o")])
    tmp = LIB + ".tmp"
    _run([HIPCC, *DEVICE, "-shared", "-fPIC", *objs, "-o", tmp, f"-Wl,-rpath,{ROCM}/lib"])
    os.replace(tmp, LIB)
    return LIB


def clean():
    shutil.rmtree(BUILD, ignore_errors=True)
    if os.path.exists(LIB):
        os.remove(LIB)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
