"""Builds libmpcg.so (HIP for gfx950 plus the host layout builder) in-tree.

Run ``python -m mixed_precision_sparse_amd.build`` or call :func:`build`.
Every call recompiles; objects go to ``_build/`` under the package.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmpcg.so")
BUILD_DIR = os.path.join(PKG, "_build")
ARCH = "gfx950"

SOURCES = ["mpcg_layout.cpp", "mpcg_reuse.cpp", "mpcg_tuning.cpp", "mpcg_runtime.hip", "mpcg_stream.hip"]

# Packed-FP32 instructions are disabled for all device code (no v_pk_*_f32).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    objs = []
    common = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
              f"-I{os.path.join(os.path.dirname(PKG), 'include')}"]
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(BUILD_DIR, src + ".o")
        if src.endswith(".hip"):
            cmd = [cc, "-x", "hip", f"--offload-arch={ARCH}", *DEVICE_FLAGS, *common, "-c", path,
                   "-o", obj]
        else:
            cmd = [cc, *common, "-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [cc, "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp, *objs, "-lpthread"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
