"""Build libvpce.so in-tree for gfx950.

The kernels and the C ABI are compiled with hipcc for gfx950 only, then linked
against the HIP runtime that PyTorch itself loads, so that the library and
torch share one runtime (and one set of streams) in a process.

    python -m vocabulary_projection_cross_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libvpce.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no packed-fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def torch_lib_dir() -> str:
    import torch  # only to locate the HIP runtime torch ships
    return os.path.join(os.path.dirname(torch.__file__), "lib")


def build(verbose: bool = False, save_temps: bool = False) -> str:
    os.makedirs(os.path.join(HERE, "_build"), exist_ok=True)
    obj = os.path.join(HERE, "_build", "vpce.o")
    src = os.path.join(CSRC, "vpce.hip")
    cmd = [HIPCC, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
    if save_temps:
        cmd.insert(1, "-save-temps=obj")
    _run(cmd, verbose)
    tl = torch_lib_dir()
    tmp = LIB + ".tmp"
    link = ["g++", "-shared", "-o", tmp, obj, "-L" + tl, "-lamdhip64",
            "-Wl,-rpath," + tl, "-Wl,--no-undefined", "-Wl,-z,defs"]
    _run(link, verbose)
    os.replace(tmp, LIB)
    return LIB


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("build step failed: " + " ".join(cmd[:2]))
    if verbose and (r.stdout or r.stderr):
        sys.stderr.write(r.stdout + r.stderr)


if __name__ == "__main__":
    print(build(verbose=True, save_temps="--save-temps" in sys.argv))
