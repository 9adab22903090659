#!/usr/bin/env python3
"""Benchmark of the DFlash draft block-attention hot path on one MI355X.

One step = one pass of the path over one synthetic batch: the per-head q/k
RMSNorm + NeoX RoPE of the block rows and the block attention over
[context; block], as one ``dflash_block_attention`` call with the fused
prologue (work-unit lookup, norm + RoPE, MFMA attention, split merge).
``--unfused`` runs ``dflash_qk_norm_rope`` in place first and the attention
on the normed rows (two calls). The context keys are prepared once
before timing (``dflash_context_kv`` / K-only ``dflash_qk_norm_rope``), as a
serving engine does when it appends context rows.

Default workload: the Qwen3-8B-shaped draft layer (8 requests, context
lengths uniform in [512, 2048], 16 block rows, Hq=32, Hkv=8, Dh=128, bf16,
bidirectional). Inputs are resident in HBM before timing; ``--rotate`` copies
of the batch are cycled so that the 256 MB Infinity Cache cannot serve the
re-reads; the steps are replayed from a HIP graph.

Prints one JSON line (rank 0).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s


def algorithmic_cost(wl):
    """Bytes and flops the attention step must move / compute (visible keys only)."""
    vis = wl.visible_keys()                               # key rows per request
    esz = 2 if wl.dtype == "bf16" else 4
    kv_row = 2 * wl.hkv * wl.dh * esz                     # K + V bytes per key row (all heads)
    qo = 2 * wl.blk_lens.astype(np.int64) * wl.hq * wl.dh * esz
    bytes_attn = int((vis * kv_row).sum() + qo.sum())
    if wl.causal:
        # each query sees only its own visible keys
        flops = 0
        for c, b in zip(wl.ctx_lens.tolist(), wl.blk_lens.tolist()):
            for i in range(b):
                qi = c + i
                lo = max(0, qi - wl.window + 1) if wl.window > 0 else 0
                flops += (qi + 1 - lo)
        flops_attn = int(flops * wl.hq * 4 * wl.dh)
    else:
        flops_attn = int((wl.blk_lens.astype(np.int64) * vis).sum() * wl.hq * 4 * wl.dh)
    # q/k norm + RoPE: read and write q and k of the block rows.
    bytes_prologue = int(2 * wl.total_blk * (wl.hq + wl.hkv) * wl.dh * esz)
    return bytes_attn, flops_attn, bytes_prologue


def source_digest() -> str:
    p = os.path.join(ROOT, "block_diffusion_draft_dflash_amd", "csrc", "block_attention.hip")
    with open(p, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def committed_traffic(workload: str):
    """HBM bytes per attention launch from the committed counter summary, if it
    was taken on the current kernel source."""
    p = os.path.join(ROOT, "profiles", f"block_attn_{workload}_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != source_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(wl, budget_s: float):
    """Time the fp64 oracle on the host on the same batch (bounded sample)."""
    from oracle import dflash_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    _, k_ctx = O.qk_norm_rope(None, wl.k_ctx, None, wl.k_norm_w, wl.ctx_positions, wl.eps,
                              wl.theta)
    reps = 0
    t0 = time.perf_counter()
    while True:
        O.draft_block_attention(wl.q, wl.k_blk, wl.v_blk, wl.blk_positions, k_ctx, wl.v_ctx,
                                wl.cu_ctx, wl.cu_blk, wl.q_norm_w, wl.k_norm_w, wl.eps, wl.theta,
                                wl.scale, wl.causal, wl.window)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return el / reps, reps, threads


def device_copy_gbs(stream, mib=512, reps=5):
    """What a plain device-to-device copy achieves on this GPU (bytes read +
    written per second), measured in the same run: the attainable stream rate
    beside the nominal 8 TB/s."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / reps
    del src, dst
    return 2.0 * n / t / 1e9


def time_layer(wl, hidden, stream, use_graph, reps=60):
    """The draft layer around the attention on this batch's block rows:
    dflash_block_qkv (input norm + merged q/k/v), the fused attention, and
    dflash_o_proj, each timed with HIP events on the launch stream over
    weight copies cycled so the last-level cache cannot serve them. Roofline:
    HBM (the weights are the bytes at these row counts)."""
    import torch
    from block_diffusion_draft_dflash_amd.pipeline import LayerPath
    from block_diffusion_draft_dflash_amd.workloads import make_layer_inputs

    li = make_layer_inputs(wl, hidden)
    t, n_qkv, in_dim = wl.total_blk, (wl.hq + 2 * wl.hkv) * wl.dh, wl.hq * wl.dh
    w_bytes = (n_qkv * hidden + hidden * in_dim) * 2
    copies = max(2, -(-(512 << 20) // max(1, w_bytes)))
    lps = [LayerPath(wl, li) for _ in range(copies)]
    for lp in lps:
        lp.step()
    torch.cuda.synchronize()

    def run(which):
        for lp in lps:
            getattr(lp, which)()

    graphs = {}
    if use_graph:
        for which in ("qkv", "o_proj", "step"):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run(which)
            graphs[which] = g
        torch.cuda.synchronize()

    def timed(which):
        go = (lambda: graphs[which].replay()) if use_graph else (lambda: run(which))
        for _ in range(3):
            go()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            go()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * len(lps))

    qkv_us, o_us, step_us = timed("qkv"), timed("o_proj"), timed("step")
    # algorithmic bytes: block_qkv reads hidden and the residual, writes the
    # residual and q/k/v, reads the norm weight and W_qkv; o_proj reads the
    # attention output and W_o and writes its output
    qkv_bytes = 3 * t * hidden * 2 + hidden * 4 + n_qkv * hidden * 2 + t * n_qkv * 2
    o_bytes = t * in_dim * 2 + hidden * in_dim * 2 + t * hidden * 2
    qkv_gbs = qkv_bytes / (qkv_us * 1e-6) / 1e9
    o_gbs = o_bytes / (o_us * 1e-6) / 1e9
    return {
        "hidden": hidden, "weight_copies": copies,
        "block_qkv": {"us": qkv_us, "bytes": qkv_bytes, "achieved_gbs": qkv_gbs,
                      "frac": qkv_gbs / HBM_PEAK_GBS, "bound": "hbm"},
        "o_proj": {"us": o_us, "bytes": o_bytes, "achieved_gbs": o_gbs,
                   "frac": o_gbs / HBM_PEAK_GBS, "bound": "hbm"},
        "layer_us": step_us,
        "layer_note": "block_qkv + dflash_block_attention (fused q/k norm + RoPE) + o_proj",
    }


def time_draft_step(wl, hidden, taps, stream, reps=50):
    """A whole propose step of one draft layer on this batch's shape, replayed
    from one HIP graph: the integer preparation, fc combine of the verified
    rows' tapped features, their context K/V appended to a paged store,
    block q/k/v, the paged attention (work split planned on the device) and
    o_proj. Each request verifies one block of rows on top of its context."""
    import numpy as np
    import torch
    from block_diffusion_draft_dflash_amd.pipeline import DraftStep

    nqpr = int(wl.blk_lens.max())
    rows = nqpr
    pages = (int(wl.ctx_lens.max()) + rows + 15) // 16 + 1
    ds = DraftStep(wl.num_reqs, nqpr, rows, hidden=hidden, taps=taps, hq=wl.hq, hkv=wl.hkv,
                   dh=wl.dh, pages_per_req=pages, seed=11)
    rng = np.random.default_rng(12)
    pos = np.concatenate([np.arange(c, c + rows) for c in wl.ctx_lens.tolist()])
    rej = rng.integers(0, rows, size=wl.num_reqs)
    ds.set_step(pos, rej, np.ones(wl.num_reqs), rng.integers(0, 1000, size=wl.num_reqs),
                rng.standard_normal((wl.num_reqs * rows, hidden * taps), dtype=np.float32))
    ds.run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ds.run()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    n_qkv = (wl.hq + 2 * wl.hkv) * wl.dh
    w_bytes = 2 * (hidden * hidden * taps + 2 * wl.hkv * wl.dh * hidden + n_qkv * hidden
                   + hidden * wl.hq * wl.dh)
    return {"us": us, "requests": wl.num_reqs, "verified_rows_per_request": rows,
            "block_rows_per_request": nqpr, "hidden": hidden, "taps": taps,
            "context_rows": int(wl.total_ctx), "weight_bytes": w_bytes,
            "stages": "prepare_inputs, fc_combine, context_kv, kv_scatter, block_qkv, "
                      "block_attention_paged (fused q/k norm + RoPE, device-planned), o_proj",
            "note": "one HIP graph replay per step; the weights (fc alone "
                    f"{hidden * hidden * taps * 2 / 1e6:.0f} MB) are read once per step"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1200)
    ap.add_argument("--warmup", type=int, default=120)
    ap.add_argument("--workload", default="qwen3_8b_draft")
    ap.add_argument("--rotate", type=int, default=12, help="copies of the batch cycled per step")
    ap.add_argument("--split-keys", type=int, default=0)
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    ap.add_argument("--unfused", action="store_true",
                    help="q/k norm + RoPE as a separate in-place call before the attention")
    ap.add_argument("--paged", action="store_true",
                    help="read the context from a paged store (dflash_block_attention_paged)")
    ap.add_argument("--device-plan", action="store_true",
                    help="leave the work split to the kernels (no host copies of the lengths)")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle time (0: skip)")
    ap.add_argument("--layer-hidden", type=int, default=4096,
                    help="hidden size of the draft layer whose projections around the attention "
                         "(dflash_block_qkv, dflash_o_proj) are also timed (0: skip)")
    ap.add_argument("--draft-step-taps", type=int, default=5,
                    help="target taps of the fc combine in the timed whole propose step (0: skip it)")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="before timing, run a plain device copy of this many MiB (3 times) so a "
                         "counter profile of the same run can scale FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not supported "
              "(sharding across GPUs is described, not built).", file=sys.stderr)
        return 2

    import torch
    from block_diffusion_draft_dflash_amd import binding as B
    from block_diffusion_draft_dflash_amd.pipeline import DevicePath
    from block_diffusion_draft_dflash_amd.workloads import make_workload

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    B.load()
    if args.copy_calibration_mb > 0:
        n = args.copy_calibration_mb << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    wl = make_workload(args.workload)
    paths = [DevicePath(wl, split_keys=args.split_keys, host_lengths=not args.device_plan,
                        paged=args.paged)
             for _ in range(args.rotate)]
    for p in paths:
        p.prepare_context()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    fused = wl.dtype == "bf16" and not args.unfused

    def run_steps(n, attention_only=False):
        for i in range(n):
            p = paths[i % len(paths)]
            if fused:
                p.step_fused()          # the step is the attention call
            elif attention_only:
                p.attention()
            else:
                p.step()

    per_graph = len(paths)
    use_graph = not args.no_graph
    if use_graph:
        # warm the launch path (function attributes, code objects) before capture
        run_steps(per_graph)
        torch.cuda.synchronize()
        g_step = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_step):
            run_steps(per_graph)
        g_attn = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_attn):
            run_steps(per_graph, attention_only=True)
        torch.cuda.synchronize()

        def steps(n, attention_only=False):
            g = g_attn if attention_only else g_step
            for _ in range(max(1, n // per_graph)):
                g.replay()
        steps_eff = max(1, args.steps // per_graph) * per_graph
    else:
        steps = run_steps
        steps_eff = args.steps

    steps(args.warmup)
    torch.cuda.synchronize()

    # ---- timed region: exactly steps_eff steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    steps(steps_eff)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / steps_eff

    # ---- dominant kernel (block attention) average duration, HIP events on its stream
    n_attn = steps_eff
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    steps(n_attn, attention_only=True)
    ev1.record(stream)
    torch.cuda.synchronize()
    attn_us = ev0.elapsed_time(ev1) * 1e3 / (max(1, n_attn // per_graph) * per_graph
                                            if use_graph else n_attn)

    bytes_attn, flops_attn, bytes_pro = algorithmic_cost(wl)
    # (skipped in a counter-calibration run, whose copy must be the only one)
    copy_gbs = device_copy_gbs(stream) if args.copy_calibration_mb == 0 else None
    step_s = ms_per_step * 1e-3
    value = flops_attn / step_s / 1e12
    tokens_per_s = wl.total_blk / step_s
    achieved_gbs = bytes_attn / (attn_us * 1e-6) / 1e9
    # the counters were taken on the default launch (packed store, fused
    # prologue, host-planned split): another launch gets no traffic figure
    default_launch = not (args.paged or args.unfused or args.device_plan or args.split_keys)
    traffic = committed_traffic(args.workload) if default_launch else None

    # Context-K/V precompute (hidden-state workloads): the dflash_context_kv
    # call (weight fold, row rms, fused GEMM + k-norm + RoPE), HIP events on
    # its stream, against the dense bf16 MFMA peak.
    ckv = None
    if wl.hidden is not None:
        p0 = paths[0]
        p0.prepare_context()
        torch.cuda.synchronize()
        reps = 5
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            p0.prepare_context()
        e1.record(stream)
        torch.cuda.synchronize()
        ckv_ms = e0.elapsed_time(e1) / reps
        ckv_flops = 2.0 * wl.total_ctx * wl.hidden_size * (2 * wl.hkv * wl.dh)
        ckv = {"ms": ckv_ms, "tflops": ckv_flops / (ckv_ms * 1e-3) / 1e12,
               "peak_tflops": BF16_PEAK_TFLOPS,
               "frac": ckv_flops / (ckv_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
               "flops": ckv_flops, "rows": wl.total_ctx, "hidden": wl.hidden_size}

    layer = None
    if args.layer_hidden > 0 and wl.dtype == "bf16" and not args.paged:
        layer = time_layer(wl, args.layer_hidden, stream, use_graph)
    draft_step = None
    if (args.draft_step_taps > 0 and args.layer_hidden > 0 and wl.dtype == "bf16"
            and not args.paged and wl.hidden is None):
        draft_step = time_draft_step(wl, args.layer_hidden, args.draft_step_taps, stream)

    cpu = None
    if args.cpu_budget > 0:
        t_cpu, reps, threads = cpu_baseline(wl, args.cpu_budget)
        cpu = {
            "value": flops_attn / t_cpu / 1e12,
            "unit": "TFLOP/s",
            "cores": threads,
            "kind": "oracle",
            "sample": (f"fp64 numpy oracle, q/k norm + RoPE + block attention over the full "
                       f"{args.workload} batch ({wl.num_reqs} requests, {wl.total_ctx} context rows, "
                       f"{wl.total_blk} block rows), {reps} passes in {t_cpu * reps:.1f} s"),
            "ms_per_step": t_cpu * 1e3,
            "draft_query_tokens_per_s": wl.total_blk / t_cpu,
        }

    rec = {
        "metric": "block-attention TFLOP/s and draft query tokens/s; % of MI355X roofline",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps_eff,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "requests": wl.num_reqs,
            "context_rows": wl.total_ctx,
            "block_rows": wl.total_blk,
            "hq": wl.hq, "hkv": wl.hkv, "dh": wl.dh,
            "mask": ("causal, window %d" % wl.window) if wl.causal else "bidirectional",
            "rotating_copies": len(paths),
            "hip_graph": use_graph,
            "fused_qk_norm_rope": fused,
            "work_split": "device-planned" if args.device_plan else "host-planned",
            "context_store": "paged (16-row pages)" if args.paged else "packed",
        },
        "draft_query_tokens_per_s": tokens_per_s,
        "roofline": {
            "bound": "hbm",
            "kernel": ("dflash_block_attention%s call = block_attn_bf16_kernel%s + "
                       "block_attn_merge_kernel" % ("_paged" if args.paged else "",
                                                    " (fused q/k norm + RoPE)" if fused else "")),
            "achieved": achieved_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved_gbs / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": bytes_attn,
            "avg_launch_us": attn_us,
            "achievable_copy_gbs": copy_gbs,
            "frac_of_copy": achieved_gbs / copy_gbs if copy_gbs else None,
        },
        "cpu_baseline": cpu,
        "context_kv": ckv,
        "draft_layer": layer,
        "draft_step": draft_step,
        "algorithmic": {"attention_bytes": bytes_attn, "attention_flops": flops_attn,
                        "prologue_bytes": bytes_pro},
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
