"""Build libqt.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libqt.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-FP32 instructions are disabled for every GPU code object: the
# compiler would otherwise form v_pk_* f32 ops from plain float code.
GPU_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I", os.path.join(ROOT, "include")]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
        raise RuntimeError("hipcc failed")


def build_library(out: str = LIB, verbose: bool = False) -> str:
    objs = []
    build_dir = os.path.join(HERE, "_build")
    os.makedirs(build_dir, exist_ok=True)
    for src, gpu in (("kernels.hip", True), ("frame.hip", True), ("api.cpp", False)):
        obj = os.path.join(build_dir, src + ".o")
        cmd = [HIPCC, *COMMON, *(GPU_FLAGS if gpu else []), "-c", os.path.join(CSRC, src), "-o", obj]
        if gpu:
            cmd[1:1] = ["-x", "hip"]
        if verbose:
            print(" ".join(cmd))
        _run(cmd)
        objs.append(obj)
    tmp = out + ".tmp"
    _run([HIPCC, "-shared", *GPU_FLAGS, "-o", tmp, *objs])
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(verbose=True))
