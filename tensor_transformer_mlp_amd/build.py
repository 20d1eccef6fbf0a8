"""Build libtpmlp.so (HIP, gfx950) and libtpsynth.so (host C) in-tree.

    python -m tensor_transformer_mlp_amd.build

hipcc cross-compiles for gfx950 without a GPU.  Device code is built with the
packed-fp32 instructions disabled (``-packed-fp32-ops``).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libtpmlp.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = [os.path.join(CSRC, "tp_mlp_kernels.hip"), os.path.join(CSRC, "tp_mlp_abi.cpp")]
DEPS = SOURCES + [os.path.join(CSRC, "tp_mlp_kernels.h"), os.path.join(INCLUDE, "tp_mlp.h")]


def hipcc_cmd(out: str, extra=()) -> list:
    return [HIPCC, "--offload-arch=" + ARCH, "-O3", "-std=c++20", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC, *extra, "-o", out, *SOURCES]


def build_lib(force: bool = True, verbose: bool = False) -> str:
    """Compile libtpmlp.so.  With force=False, only when a source is newer."""
    if not force and os.path.exists(LIB):
        t = os.path.getmtime(LIB)
        if all(os.path.getmtime(d) <= t for d in DEPS):
            return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = hipcc_cmd(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


def build_all(verbose: bool = False) -> None:
    from . import inputs
    inputs.build_synth(force=True)
    build_lib(force=True, verbose=verbose)


if __name__ == "__main__":
    build_all(verbose=True)
    print("built", LIB, file=sys.stderr)
