"""The library's host code (argument checks, work planners, launch setup) built
with AddressSanitizer and UndefinedBehaviorSanitizer on the host side only
(device code is compiled as usual and never runs here), then driven through
every entry point by host_sanitizer_driver.py in a child process with the
sanitizer runtime preloaded. Any out-of-bounds access, use of freed memory or
undefined behaviour in that code aborts the child with a report. The child
sees no GPU (its device pointers are fake), so this runs on the CPU only.
"""
import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_diffusion_draft_dflash_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "host_sanitizers")
SOURCES = ["dflash_api.hip", "rope_qknorm.hip", "block_attention.hip", "context_kv.hip",
           "kv_store.hip", "layer_proj.hip", "propose_prep.hip", "noalloc_scratch.hip"]
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all"]


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_host_code_under_asan_and_ubsan():
    hipcc, rt = _hipcc(), _asan_runtime()
    if hipcc is None or rt is None:
        pytest.skip("hipcc or the clang sanitizer runtime is not installed")
    os.makedirs(OUT, exist_ok=True)
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-w",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC] + SAN

    def compile_one(src):
        obj = os.path.join(OUT, src.replace(".hip", ".o"))
        subprocess.run([hipcc, *flags, "-c", os.path.join(CSRC, src), "-o", obj], check=True,
                       capture_output=True)
        return obj

    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    lib = os.path.join(OUT, "libdflash_sanitized.so")
    subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *SAN[:4], "-shared-libasan",
                    *objs, "-o", lib], check=True, capture_output=True)
    # no device may be visible to the child: its calls carry fake device pointers
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="-1",
               ROCR_VISIBLE_DEVICES="-1", CUDA_VISIBLE_DEVICES="-1")
    res = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "host_sanitizer_driver.py"), lib,
                          ROOT], env=env, capture_output=True, text=True, timeout=600)
    if res.returncode == 3 and "GPU is visible" in res.stdout:
        pytest.skip("a GPU is visible to the child process; the driver runs on machines without one")
    assert res.returncode == 0, (res.stdout[-3000:], res.stderr[-6000:])
    assert "no report" in res.stdout
    assert "ERROR: AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr
