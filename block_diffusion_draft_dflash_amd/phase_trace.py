"""Per-workgroup phase timing of dflash_block_attention (diagnostic build).

Usage: ``python -m block_diffusion_draft_dflash_amd.phase_trace [workload ...]``
(default: ctx_kv qwen3_8b_draft large_decode swa), on a GPU, after the build
has linked ``libdflash_phasetrace.so`` (the library with the attention
compiled with -DDFLASH_PHASE_TRACE). Every workgroup of the main and the merge
kernel records the GPU's 100 MHz real-time counter at its start, after the
unit lookup, at the start and end of its tile loop and at its end, plus its
XCD; the records sit at the end of the workspace. Each call (the fused q/k
norm + RoPE form, host-planned split, as bench.py times it) runs on one of
several copies of the batch, cycled so that the context K/V comes from HBM;
the first round of calls is discarded. Times are microseconds from the
call's first workgroup start; per-call medians over workgroups, then the
median over calls.
"""
from __future__ import annotations

import ctypes
import os
import statistics
import sys

import numpy as np

from . import binding as B
from .build import TRACE_LIB

ROTATE_BYTES = 512 << 20


def _layout(lib, params):
    lib.dflash_phase_trace_layout.restype = ctypes.c_size_t
    lib.dflash_phase_trace_layout.argtypes = [ctypes.POINTER(B.BlockAttnParams), ctypes.c_int,
                                              ctypes.POINTER(ctypes.c_int64),
                                              ctypes.POINTER(ctypes.c_int64)]
    nm, ng = ctypes.c_int64(), ctypes.c_int64()
    off = lib.dflash_phase_trace_layout(ctypes.byref(params), 0, ctypes.byref(nm), ctypes.byref(ng))
    return int(off), int(nm.value), int(ng.value)


def _med(x):
    return float(statistics.median(x)) if len(x) else float("nan")


def trace_workload(name: str, calls: int = 12):
    import torch
    from .pipeline import DevicePath
    from .workloads import make_workload

    lib = B.load(TRACE_LIB)
    if not hasattr(lib, "dflash_phase_trace_layout"):
        raise RuntimeError("the product library is loaded in this process; phase_trace needs "
                           "libdflash_phasetrace.so loaded first")
    wl = make_workload(name)
    kv_bytes = int(wl.visible_keys().sum()) * 2 * wl.hkv * wl.dh * 2
    copies = max(2, -(-ROTATE_BYTES // max(1, kv_bytes)))
    paths = [DevicePath(wl) for _ in range(copies)]
    for p in paths:
        p.prepare_context()
    off, nmain, nmerge = _layout(lib, paths[0].params)
    rows = []
    for i in range(copies + calls):
        p = paths[i % copies]
        region = p.ws[off:off + 64 * (nmain + nmerge)]
        region.zero_()
        p.attention_fused()
        torch.cuda.synchronize()
        if i < copies:
            continue
        rec = region.view(torch.int64).cpu().numpy().reshape(-1, 8)
        rows.append(rec)
    per_call = []
    for rec in rows:
        main = rec[rec[:, 7] == 1]
        merge = rec[rec[:, 7] == 2]
        t0 = main[:, 0].min()
        us = lambda x: (x - t0) / 100.0
        d = {
            "wgs": len(main), "merge_wgs": len(merge),
            "lookup": _med((main[:, 1] - main[:, 0]) / 100.0),
            "prologue": _med((main[:, 2] - main[:, 1]) / 100.0),
            "loop": _med((main[:, 3] - main[:, 2]) / 100.0),
            "epilogue": _med((main[:, 4] - main[:, 3]) / 100.0),
            "us_per_tile": _med((main[:, 3] - main[:, 2]) / 100.0 / np.maximum(main[:, 6], 1)),
            "start_spread": float(us(main[:, 0]).max()),
            "wg_end_median": _med(us(main[:, 4])),
            "main_end": float(us(main[:, 4]).max()),
        }
        if len(merge):
            d["merge_start"] = float(us(merge[:, 0]).min())
            d["merge_end"] = float(us(merge[:, 4]).max())
            d["gap"] = d["merge_start"] - d["main_end"]
            d["merge"] = d["merge_end"] - d["merge_start"]
        else:
            d.update(merge_start=float("nan"), merge_end=d["main_end"], gap=0.0, merge=0.0)
        xe = [_med(us(main[main[:, 5] == x][:, 4])) for x in range(8) if (main[:, 5] == x).any()]
        d["xcd_end_min"], d["xcd_end_max"] = min(xe), max(xe)
        per_call.append(d)
    keys = per_call[0].keys()
    return {k: _med([c[k] for c in per_call]) for k in keys}, copies, len(per_call)


COLUMNS = [("wgs", "main WGs", "{:.0f}"), ("merge_wgs", "merge WGs", "{:.0f}"),
           ("lookup", "lookup", "{:.2f}"), ("prologue", "prologue + first tiles", "{:.2f}"),
           ("loop", "tile loop", "{:.2f}"), ("us_per_tile", "us / tile", "{:.2f}"),
           ("epilogue", "epilogue", "{:.2f}"), ("start_spread", "last WG start", "{:.2f}"),
           ("wg_end_median", "WG end (median)", "{:.2f}"),
           ("xcd_end_min", "XCD median end (min)", "{:.2f}"),
           ("xcd_end_max", "XCD median end (max)", "{:.2f}"), ("main_end", "main kernel end", "{:.2f}"),
           ("gap", "gap to merge", "{:.2f}"), ("merge", "merge kernel", "{:.2f}"),
           ("merge_end", "call end", "{:.2f}")]


def main(argv) -> int:
    import torch
    if not torch.cuda.is_available():
        print("phase_trace: no GPU visible", file=sys.stderr)
        return 1
    if not os.path.exists(TRACE_LIB):
        print(f"phase_trace: {TRACE_LIB} is missing (run the build)", file=sys.stderr)
        return 1
    names = argv or ["ctx_kv", "qwen3_8b_draft", "large_decode", "swa"]
    res = []
    for n in names:
        r, copies, ncalls = trace_workload(n)
        print(f"{n}: {ncalls} calls over {copies} copies", flush=True)
        res.append((n, r))
    print()
    print("| phase (us) | " + " | ".join(n for n, _ in res) + " |")
    print("|---|" + "---|" * len(res))
    for k, label, fmt in COLUMNS:
        print(f"| {label} | " + " | ".join(fmt.format(r[k]) for _, r in res) + " |")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
