"""Builds libfa.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

    python -m exact_io_aware_64_amd.build

Every call recompiles.  Objects go to ``_build/`` at the repository root; the
shared library lands next to this file, where the binding loads it.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")
ARCH = "gfx950"

SOURCES = ["fa_api.hip", "fa_fwd_bf16.hip", "fa_bwd_bf16.hip", "fa_bwd_bf16_d128.hip",
           "fa_fwd_f32.hip", "fa_bwd_f32.hip"]

# Packed fp32 instructions are disabled for all device code: the compiler
# would otherwise pair independent fp32 operations into them.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
BASE_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
              "-Wno-unused-command-line-argument"] + DEVICE_FLAGS
# MFMA accumulators in the architectural VGPRs: the kernels that run two or
# more waves per SIMD fit their 256 registers that way.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
# Per-source flags.  The d = 128 backward runs one wave per SIMD and keeps its
# accumulators in the accumulation registers; its 64-slot tile loop is past
# the default limit for fully unrolling a loop.
UNROLL = ["-mllvm", "-pragma-unroll-threshold=200000"]
SOURCE_FLAGS = {
    "fa_bwd_bf16_d128.hip": UNROLL,
    # the d = 128 dropout forward's 32-slot tile loop needs the same limit
    "fa_fwd_bf16.hip": VGPR_FORM + UNROLL,
}


def source_flags(src: str) -> list:
    """The compiler flags of one source file."""
    return BASE_FLAGS + SOURCE_FLAGS.get(src, VGPR_FORM)


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libfa.so")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *source_flags(src), "-Rpass-analysis=kernel-resource-usage",
           "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    lines = [l for l in r.stderr.splitlines() if noise not in l]
    usage = [l for l in lines if "kernel-resource-usage" in l]
    err = "\n".join(l for l in lines if "kernel-resource-usage" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    # A kernel that spills or calls an out-of-line function uses scratch
    # memory, which costs far more than any register it saves: refuse it.
    for l in usage:
        if "ScratchSize" in l and not l.rstrip().endswith(": 0 [-Rpass-analysis=kernel-resource-usage]"):
            raise RuntimeError(f"{src}: a kernel uses scratch memory:\n{l}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
