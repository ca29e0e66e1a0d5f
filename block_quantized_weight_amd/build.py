"""Build libqgemv.so (HIP for gfx950) in-tree with hipcc.

Every HIP translation unit is compiled with packed-FP32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops); the host pass warns that it does
not know the feature, which is harmless.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libqgemv.so")
BUILD_DIR = os.path.join(ROOT, "_build", "qgemv")
ARCH = "gfx950"

SOURCES = ["api.cpp", "select.cpp", "kernels_vector.hip", "kernels_mfma.hip", "scratch.hip", "sweep.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I" + os.path.join(ROOT, "include")]
DEVICE = ["-x", "hip", "--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the qgemv library needs ROCm's hipcc to build")


def _compile(src: str) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD_DIR, src + ".o")
    cmd = [hipcc(), "-c"] + COMMON
    if src.endswith(".hip"):
        cmd += DEVICE
    else:
        cmd += ["-D__HIP_PLATFORM_AMD__"]
    cmd += [path, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


READ_CONTROL_SRC = "read_control.hip"
READ_CONTROL_OUT = os.path.join(PKG, "libreadctl.so")


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link libqgemv.so next to this file, and the benchmark's
    plain-read control (libreadctl.so, a separate library the GEMV never loads)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES + [READ_CONTROL_SRC]))
    _link(objs[:-1], OUT)
    _link(objs[-1:], READ_CONTROL_OUT)
    if verbose:
        print("built", OUT, "and", READ_CONTROL_OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True, jobs=int(sys.argv[1]) if len(sys.argv) > 1 else 8)
