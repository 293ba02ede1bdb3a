"""Build libfa.so (gfx950 only) in-tree with hipcc.

    python -m io_aware_tiled_amd.build          # from the repository root

Sources are compiled in parallel into io_aware_tiled_amd/_build/ and linked
into io_aware_tiled_amd/libfa.so.  Every HIP source is compiled with packed
FP32 instructions disabled (-packed-fp32-ops).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfa.so")
ARCH = "gfx950"

SOURCES = ["fa_fwd.hip", "fa_bwd.hip", "fa_fp8.hip", "fa_linear.hip",
           "fa_noalloc.hip", "fa_api.cpp"]

# Per-source flags.  The VALU reads the score MFMAs' results, so MFMA
# results are kept in VGPRs rather than AGPRs (which the VALU can only reach
# through copies); the backward's long-lived dK/dV accumulators are placed in
# AGPRs explicitly.
SOURCE_FLAGS = {"fa_fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "fa_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "fa_fp8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "fa_linear.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found; the HIP toolchain is required")
    return p


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, *SOURCE_FLAGS.get(src, []), *extra, "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


MICRO_SRC = os.path.join(ROOT, "microbench", "micro.hip")
MICRO_LIB = os.path.join(ROOT, "microbench", "libmicro.so")


def build_micro(verbose: bool = False) -> str:
    """Compile the microbenchmark library (not part of libfa) that
    bench.py --micro drives."""
    tmp = MICRO_LIB + ".tmp"
    cmd = [hipcc(), *COMMON, "-shared", MICRO_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for micro.hip:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, MICRO_LIB)
    if verbose:
        print(f"built {MICRO_LIB}")
    return MICRO_LIB


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile every source and link libfa.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    extra = list(extra or [])
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs,
           "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
    build_micro(verbose=True)
