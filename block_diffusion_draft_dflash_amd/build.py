"""Build libdflash.so in-tree with hipcc for gfx950.

Usage: ``python -m block_diffusion_draft_dflash_amd.build``. Every call
recompiles every source (objects go to ``_build/`` at the repository root,
the library next to this file). It also links libdflash_phasetrace.so, the
same library with the block attention compiled with -DDFLASH_PHASE_TRACE
(per-workgroup phase timestamps; read by ``phase_trace.py``, never by the
product path).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdflash.so")
TRACE_LIB = os.path.join(PKG, "libdflash_phasetrace.so")
TRACE_SOURCE = "block_attention.hip"
SOURCES = ["dflash_api.hip", "rope_qknorm.hip", "block_attention.hip", "context_kv.hip",
           "kv_store.hip", "layer_proj.hip", "propose_prep.hip", "noalloc_scratch.hip"]
ARCH = "gfx950"

# Packed-FP32 instructions are disabled for every HIP translation unit.
HIPFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]
# Keep MFMA accumulators in VGPRs (the attention's softmax rescale and the
# projections' epilogues touch them); the context GEMM's 256 accumulators per
# lane live in the accumulation registers instead.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
AGPR_ACC_SOURCES = {"context_kv.hip"}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libdflash)")


def _compile(src: str, verbose: bool, trace: bool = False) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ("_phasetrace.o" if trace else ".o"))
    extra = [] if src in AGPR_ACC_SOURCES else VGPR_FORM
    if trace:
        extra = extra + ["-DDFLASH_PHASE_TRACE"]
    cmd = [_hipcc(), *HIPFLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def _link(objs, out: str, verbose: bool) -> None:
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(s, False) for s in SOURCES] + [(TRACE_SOURCE, True)]
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], verbose, j[1]), jobs))
    _link(objs[:len(SOURCES)], LIB, verbose)
    trace_objs = [o if s != TRACE_SOURCE else objs[-1] for s, o in zip(SOURCES, objs)]
    _link(trace_objs, TRACE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
