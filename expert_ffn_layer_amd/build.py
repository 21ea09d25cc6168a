"""Build libmoe.so (HIP, gfx950) in-tree with hipcc.

    python -m expert_ffn_layer_amd.build
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["router.hip", "permute.hip", "ffn.hip", "combine.hip", "mxfp8.hip", "noalloc.hip",
           "moe_api.cpp"]

# A second build of the same sources with the heavy kernels' grid capped at 16
# blocks, so each block runs many work items in a row: the tests compare its
# bits with the default build's to cover the cross-tile paths on small shapes.
GRID16_LIB = os.path.join(PKG, "libmoe_grid16.so")
GRID16_FLAGS = ["-DMOE_HEAVY_MAX_GRID=16"]
# The same with the down GEMM's y written from registers instead of staged
# through LDS: the build in which the down GEMM's cross-tile prefetch runs
# (staging and the prefetch need the same LDS, so the default build stages).
GRID16_NS_LIB = os.path.join(PKG, "libmoe_grid16_ns.so")
GRID16_NS_FLAGS = ["-DMOE_HEAVY_MAX_GRID=16", "-DMOE_HEAVY_STAGED_EPI=0"]
# Test variant: the light loop as one persistent gate|up -> down launch
# (off in the default build; kept correct by tests/test_gpu_fused_light.py).
FUSED_LIB = os.path.join(PKG, "libmoe_fusedlight.so")
FUSED_FLAGS = ["-DMOE_FUSED_LIGHT=1"]

# -packed-fp32-ops off: packed fp32 VALU forms are not emitted.
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str, objdir: str = OBJDIR, extra=()) -> str:
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    cp = subprocess.run(cmd, capture_output=True, text=True)
    if cp.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{cp.stdout}\n{cp.stderr}")
    return obj


def build(verbose: bool = False, out: str = LIB, objdir: str = OBJDIR, extra=()) -> str:
    """Compile every source and link ``out``.  ``extra`` adds compiler flags
    (e.g. -D overrides of the kernels' compile-time tunables)."""
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(objdir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, objdir, extra), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    cp = subprocess.run(cmd, capture_output=True, text=True)
    if cp.returncode != 0:
        raise RuntimeError(f"link failed:\n{cp.stdout}\n{cp.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


def build_all(verbose: bool = False) -> None:
    """The library and its test variants (grid-capped heavy kernels with the
    down GEMM's y staged and unstaged, fused light loop)."""
    build(verbose=verbose)
    build(verbose=verbose, out=GRID16_LIB, objdir=os.path.join(OBJDIR, "grid16"),
          extra=GRID16_FLAGS)
    build(verbose=verbose, out=GRID16_NS_LIB, objdir=os.path.join(OBJDIR, "grid16_ns"),
          extra=GRID16_NS_FLAGS)
    build(verbose=verbose, out=FUSED_LIB, objdir=os.path.join(OBJDIR, "fused"),
          extra=FUSED_FLAGS)


if __name__ == "__main__":
    build_all(verbose=True)
