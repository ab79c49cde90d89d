"""Builds libverify_attn.so (the HIP kernels and the C ABI) in-tree for gfx950."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libverify_attn.so")
SOURCES = ["capi.cpp", "verify_simple.hip", "verify_mfma.hip", "verify_combine.hip",
           "tree_ops.hip", "static_scratch.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-mcode-object-version=5", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    # keep the compiler from forming packed fp32 ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix instructions written by the compiler keep their accumulators in VGPRs; the
    # partial kernel's output accumulators are placed in AGPRs by hand
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I" + os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


AB_SOURCE = "single_launch_ab.hip"  # a separate measurement library, not the verify library
AB_LIB = os.path.join(HERE, "libsingle_launch_ab.so")


PROBE_SOURCE = "lds_mfma_probe.hip"  # a separate measurement library
PROBE_LIB = os.path.join(HERE, "liblds_mfma_probe.so")


def _build_one(source: str, lib: str) -> str:
    tmp = lib + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, os.path.join(CSRC, source), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stderr[-8000:]}")
    os.replace(tmp, lib)
    return lib


def build_ab(verbose: bool = False) -> str:
    """Builds the single-launch A/B measurement library (bench.py --single-launch-ab)."""
    return _build_one(AB_SOURCE, AB_LIB)


def build_probe(verbose: bool = False) -> str:
    """Builds the LDS/matrix-core probe library (bench.py --lds-probe)."""
    return _build_one(PROBE_SOURCE, PROBE_LIB)


def build(verbose: bool = False, extra=()) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stderr[-8000:]}")
    if verbose and r.stderr.strip():
        print(r.stderr[-4000:], file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_ab())
    print(build_probe())
