"""Build libconvt.so (the C-ABI HIP library) in-tree for gfx950 with hipcc.

Every HIP source is compiled with packed-FP32 instruction selection switched
off (-Xclang -target-feature -Xclang -packed-fp32-ops).  The sources under
csrc/ link into libconvt.so next to this file; calib/calib.hip (bandwidth and
matrix-core calibration kernels for the measurements) links into
libconvt_calib.so beside it.  Run as a script or call build().
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libconvt.so")
# measurement-only calibration kernels (bench.py), outside the product library
CALIB_SRC = os.path.join(PKG, "calib", "calib.hip")
CALIB_LIB = os.path.join(PKG, "libconvt_calib.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-I", INCLUDE, "-I", CSRC]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    if src == CALIB_SRC:
        obj = os.path.join(OBJDIR, "calib_" + os.path.basename(src) + ".o")
    cmd = [HIPCC, "-c", *COMMON]
    if src.endswith(".hip"):
        cmd += ["-x", "hip", *DEVICE]
    cmd += ["-o", obj, src]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + 1)) as ex:
        objs = list(ex.map(_compile, srcs + [CALIB_SRC]))
    for lib, lib_objs in ((LIB, objs[:-1]), (CALIB_LIB, objs[-1:])):
        tmp = lib + ".tmp"
        cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *lib_objs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        os.replace(tmp, lib)
        if verbose:
            print(f"built {lib}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
