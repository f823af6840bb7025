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


BUILD_DIR = os.path.join(HERE, "_build")
PROBE = os.path.join(BUILD_DIR, "exchange_probe")


def build_library(out: str = LIB, verbose: bool = False) -> str:
    """libqt.so from the three sources (compiled in parallel), and the
    exchange-latency probe program beside the objects."""
    from concurrent.futures import ThreadPoolExecutor

    os.makedirs(BUILD_DIR, exist_ok=True)
    cmds, objs = [], []
    for src, gpu in (("kernels.hip", True), ("frame.hip", True), ("api.cpp", False)):
        obj = os.path.join(BUILD_DIR, src + ".o")
        cmd = [HIPCC, *COMMON, *(GPU_FLAGS if gpu else []), "-c", os.path.join(CSRC, src), "-o", obj]
        if gpu:
            cmd[1:1] = ["-x", "hip"]
        cmds.append(cmd)
        objs.append(obj)
    cmds.append([HIPCC, "-x", "hip", "-O3", "-std=c++17", *GPU_FLAGS, os.path.join(HERE, "exchange_probe.hip"),
                 "-o", PROBE + ".tmp"])
    if verbose:
        for c in cmds:
            print(" ".join(c))
    with ThreadPoolExecutor(len(cmds)) as ex:
        list(ex.map(_run, cmds))
    os.replace(PROBE + ".tmp", PROBE)
    tmp = out + ".tmp"
    _run([HIPCC, "-shared", *GPU_FLAGS, "-o", tmp, *objs])
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(verbose=True))
