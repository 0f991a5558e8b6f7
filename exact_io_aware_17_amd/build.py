"""Build libfa.so (the C-ABI attention library) in-tree for gfx950.

    python -m exact_io_aware_17_amd.build

Compiles every source under csrc/ with hipcc for --offload-arch=gfx950 into
exact_io_aware_17_amd/_build/, then links exact_io_aware_17_amd/libfa.so, and
links the matrix-core rate probe (csrc/probe/) into libfa_probe.so, a
separate library that only the benchmark loads. Always recompiles (it is also
the "does it build" check on machines without a GPU, where hipcc
cross-compiles).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfa.so")
PROBE_LIB = os.path.join(HERE, "libfa_probe.so")

SOURCES = ["fa_api.cpp", "fa_plan.cpp", "fa_fwd.hip", "fa_fwd_f32.hip", "fa_bwd.hip",
           "fa_noalloc.hip"]
PROBE_SOURCES = ["probe/fa_probe.hip"]

# Per-source extra flags. The 16-bit forward keeps its MFMA accumulators in
# VGPRs (its rare rescale multiplies them with VALU instructions, which cannot
# read AGPRs).
EXTRA = {"fa_fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

ARCH = "gfx950"
COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # Never form packed-fp32 VALU instructions (v_pk_*_f32).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfa)")


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.splitext(os.path.basename(src))[0] + ".o")
    cmd = ([hipcc()] + COMMON + EXTRA.get(src, []) + list(extra)
           + ["-c", os.path.join(CSRC, src), "-o", obj])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objs + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False, extra=()) -> str:
    """Compile all sources, link libfa.so and libfa_probe.so; returns the
    path of libfa.so."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
