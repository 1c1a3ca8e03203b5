"""Builds libfmha_mqa.so in-tree for gfx950 with hipcc.

    python fmha_mqa_fwd_amd/build.py        (or __graft_entry__.build())

(run by path: importing the package loads the library this builds).

Each translation unit is compiled to an object in parallel, then linked into
``fmha_mqa_fwd_amd/libfmha_mqa.so``.  The library is written to a temporary
name and renamed, so a failed build never leaves a half-written library.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_NAME = "libfmha_mqa.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["api.hip", "fmha_fwd.hip", "fmha_chunk.hip", "lse_merge.hip", "fmha_indexer.hip",
           "gather_floor.hip", "fmha_hd512.hip", "measure.hip"]
ARCH = "gfx950"

# Packed-FP32 VALU forms are kept out of the generated code on purpose; the
# host pass warns that it does not know the feature, which is harmless.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-source additions: MFMA results in ordinary VGPRs.  In the kernels that
# run at one wave per SIMD (head dim 256 and 512, the whole-chunk split
# kernel) the compiler otherwise keeps O in accumulation registers and copies
# it out and back on every tile for the (rare) rescale's multiplies; the
# other kernels of these files compile to the same code either way.
_VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
SOURCE_FLAGS = {"fmha_hd512.hip": _VGPR_FORM, "fmha_fwd.hip": _VGPR_FORM,
                "fmha_chunk.hip": _VGPR_FORM}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every HIP source and link the shared library; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([hipcc, *COMMON_FLAGS, *SOURCE_FLAGS.get(src, []), "-c",
                     os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(cmds)))) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
