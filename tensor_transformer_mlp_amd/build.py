"""Build libtpmlp.so (HIP, gfx950) and libtpsynth.so (host C) in-tree.

    python -m tensor_transformer_mlp_amd.build

hipcc cross-compiles for gfx950 without a GPU.  Device code is built with the
packed-fp32 instructions disabled (``-packed-fp32-ops``).
"""
from __future__ import annotations

import concurrent.futures
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

SOURCES = [os.path.join(CSRC, f) for f in (
    "gemm_bf16_nn.hip", "gemm_bf16_nt.hip", "gemm_bf16_tn.hip", "gemm_bf16.hip", "gemm_f32.hip",
    "reduce.hip", "transpose.hip", "attention.hip", "noalloc.hip", "tp_mlp_abi.cpp")]
HEADERS = [os.path.join(CSRC, f) for f in ("device_common.h", "gemm_bf16_impl.h", "tp_mlp_kernels.h")]
DEPS = SOURCES + HEADERS + [os.path.join(INCLUDE, "tp_mlp.h"), os.path.join(INCLUDE, "tp_mlp_dev.h")]
OBJDIR = os.path.join(HERE, "_build")

# -std=c++20: the kernels use templated lambdas.  -packed-fp32-ops: no packed
# fp32 instructions in device code.
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++20", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


# Per-source flags.  attention.hip: MFMA accumulators in ordinary VGPRs (the
# softmax reads and rescales them with VALU instructions every key block; in
# AGPRs each of those needs a copy out and back).
SOURCE_FLAGS = {"attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc_compile_cmd(src: str, obj: str) -> list:
    extra = SOURCE_FLAGS.get(os.path.basename(src), [])
    return [HIPCC, *FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-c", "-o", obj, src]


def hipcc_link_cmd(objs, out: str) -> list:
    return [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", out, *objs]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)


def build_lib(force: bool = True, verbose: bool = False) -> str:
    """Compile libtpmlp.so (each source in parallel, then one link).  With
    force=False, only when a source or header is newer than the library."""
    if not force and os.path.exists(LIB):
        t = os.path.getmtime(LIB)
        if all(os.path.getmtime(d) <= t for d in DEPS):
            return LIB
    os.makedirs(OBJDIR, exist_ok=True)
    objs = [os.path.join(OBJDIR, os.path.basename(src) + ".%d.o" % os.getpid()) for src in SOURCES]
    jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with concurrent.futures.ThreadPoolExecutor(jobs) as pool:
        list(pool.map(lambda so: _run(hipcc_compile_cmd(*so), verbose), zip(SOURCES, objs)))
    tmp = LIB + ".tmp%d" % os.getpid()
    try:
        _run(hipcc_link_cmd(objs, tmp), verbose)
        os.replace(tmp, LIB)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return LIB


def build_all(verbose: bool = False) -> None:
    from . import inputs
    inputs.build_synth(force=True)
    build_lib(force=True, verbose=verbose)


if __name__ == "__main__":
    build_all(verbose=True)
    print("built", LIB, file=sys.stderr)
