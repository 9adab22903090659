#!/usr/bin/env python3
"""Benchmark of the DFlash draft block-attention hot path on one MI355X.

One step = one draft step of the path over one synthetic batch whose context
keys and values are already resident: the per-head q/k RMSNorm + NeoX RoPE of
the block rows and the block attention over [context; block], as one
``dflash_block_attention`` call with the fused prologue (work-unit lookup,
norm + RoPE, MFMA attention, split merge). ``--unfused`` runs
``dflash_qk_norm_rope`` in place first and the attention on the normed rows
(two calls).

Default workload: ``ctx_kv`` -- 4 requests of 32768 context rows given as
hidden states [131072, 4096]; ``dflash_context_kv`` (hidden RMSNorm, K/V
projection, k-norm, RoPE) turns them into the context K/V caches before the
timed steps, as a serving engine does when it appends context rows, and is
timed in the same run (``context_kv``, against the bf16 MFMA peak), as is one
whole pass of precompute + attention (``full_pass``). The other bf16
workloads are timed in the same run as sub-records (``configs``); the draft
layer around the attention and a whole captured propose step are timed on
the Qwen3-8B-shaped batch.

Inputs are resident in HBM before timing; enough copies of each batch are
cycled that the 256 MB Infinity Cache cannot serve the re-reads; the steps
are replayed from HIP graphs, exactly ``--steps`` of them in the timed
region (whole-batch graphs plus single-step graphs for the remainder).

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
ROTATE_BYTES = 512 << 20       # bytes the rotating copies of a batch span at least
SUB_CONFIGS = ("qwen3_8b_draft", "large_decode", "swa")


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


def host_cpu():
    """(threads the oracle's BLAS uses, cores this process may run on, CPU model)."""
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    try:
        avail = len(os.sched_getaffinity(0))
    except Exception:  # pragma: no cover
        avail = os.cpu_count() or 1
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    return threads, avail, model


def _ctx_kv_sample(wl, rows):
    """The oracle's context K/V of request 0's first ``rows`` context rows
    (hidden-state workloads), with the lengths of that one-request sample."""
    from oracle import dflash_oracle as O
    from block_diffusion_draft_dflash_amd.workloads import bf16_bits_to_f32
    c0 = int(wl.cu_ctx[0])
    rows = min(rows, int(wl.ctx_lens[0]))
    hid = bf16_bits_to_f32(wl.hidden[c0:c0 + rows])
    t0 = time.perf_counter()
    k_ctx, v_ctx = O.context_kv(hid, wl.hidden_norm_w, bf16_bits_to_f32(wl.w_k),
                                bf16_bits_to_f32(wl.w_v), wl.k_norm_w,
                                wl.ctx_positions[c0:c0 + rows], wl.hkv, wl.dh, wl.eps, wl.theta)
    t_ckv = time.perf_counter() - t0
    return k_ctx, v_ctx, rows, t_ckv


def cpu_baseline(wl, budget_s: float, sample_reqs=None, ctx_rows=None):
    """Time the fp64 oracle on the host on a bounded sample of the batch.

    The sample is the first ``sample_reqs`` requests (all when None). For a
    workload given as hidden states, the oracle first builds the sample's
    context K/V itself (``context_kv`` on request 0's first ``ctx_rows`` rows,
    timed apart) and the attention pass then runs over that request alone.
    Returns a dict: seconds per attention pass, passes, threads, the sample's
    algorithmic flops and query rows, a description, and the context-K/V
    seconds and rows when built."""
    from oracle import dflash_oracle as O
    threads, avail, model = host_cpu()
    if wl.hidden is not None:
        k_ctx, v_ctx, rows, t_ckv = _ctx_kv_sample(wl, ctx_rows or int(wl.ctx_lens[0]))
        b0, b1 = int(wl.cu_blk[0]), int(wl.cu_blk[1])
        q, kb, vb, bpos = wl.q[b0:b1], wl.k_blk[b0:b1], wl.v_blk[b0:b1], wl.blk_positions[b0:b1]
        cu_ctx, cu_blk = np.array([0, rows]), np.array([0, b1 - b0])
        blk_lens = np.array([b1 - b0])
        vis = np.array([rows + (b1 - b0)])
        desc = (f"request 0 of {wl.num_reqs}: its first {rows} context rows through the oracle's "
                f"context_kv ({t_ckv:.1f} s, not in the attention time), then q/k norm + RoPE + "
                f"block attention of its {b1 - b0} block rows over them")
        ckv = {"seconds": t_ckv, "rows": rows,
               "flops": 2.0 * rows * wl.hidden_size * 2 * wl.hkv * wl.dh}
    else:
        nreq = wl.num_reqs if sample_reqs is None else min(sample_reqs, wl.num_reqs)
        c1, b1 = int(wl.cu_ctx[nreq]), int(wl.cu_blk[nreq])
        _, k_ctx = O.qk_norm_rope(None, wl.k_ctx[:c1], None, wl.k_norm_w, wl.ctx_positions[:c1],
                                  wl.eps, wl.theta)
        v_ctx = wl.v_ctx[:c1]
        q, kb, vb, bpos = wl.q[:b1], wl.k_blk[:b1], wl.v_blk[:b1], wl.blk_positions[:b1]
        cu_ctx, cu_blk = wl.cu_ctx[:nreq + 1], wl.cu_blk[:nreq + 1]
        blk_lens = wl.blk_lens[:nreq]
        vis = wl.visible_keys()[:nreq]
        desc = (f"{nreq} of {wl.num_reqs} requests ({c1} context rows, {b1} block rows): "
                "q/k norm + RoPE + block attention")
        ckv = None
    reps = 0
    t0 = time.perf_counter()
    while True:
        O.draft_block_attention(q, kb, vb, bpos, k_ctx, v_ctx, cu_ctx, cu_blk, wl.q_norm_w,
                                wl.k_norm_w, wl.eps, wl.theta, wl.scale, wl.causal, wl.window)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    if wl.causal:
        # per query its own visible keys (context + block rows at or before it, in the window)
        flops = 0
        for r in range(len(blk_lens)):
            c = int(cu_ctx[r + 1] - cu_ctx[r])
            for i in range(int(blk_lens[r])):
                qi = c + i
                lo = max(0, qi - wl.window + 1) if wl.window > 0 else 0
                flops += qi + 1 - lo
        flops *= wl.hq * 4 * wl.dh
    else:
        flops = int((blk_lens.astype(np.int64) * vis).sum()) * wl.hq * 4 * wl.dh
    return {"seconds": el / reps, "passes": reps, "threads": threads, "cores_available": avail,
            "cpu_model": model, "flops": flops, "query_rows": int(blk_lens.sum()),
            "sample": desc, "context_kv": ckv}


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


class StepRunner:
    """Steps of the path over ``copies`` resident copies of one batch, replayed
    from HIP graphs: one graph holds a step on every copy in turn, and one
    graph per copy holds a single step, so that any number of steps runs
    exactly (whole passes over the copies, then single steps)."""

    def __init__(self, paths, fused, use_graph):
        import torch
        self.paths, self.fused, self.use_graph = paths, fused, use_graph
        if not use_graph:
            return
        for i in range(len(paths)):          # warm the launch path before capture
            self._step(i)
        torch.cuda.synchronize()
        self.g_all = {}
        self.g_one = {}
        for attn_only in (False, True):
            if self.fused and attn_only:
                self.g_all[True], self.g_one[True] = self.g_all[False], self.g_one[False]
                break
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(len(paths)):
                    self._step(i, attn_only)
            self.g_all[attn_only] = g
            ones = []
            for i in range(len(paths)):
                g1 = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g1):
                    self._step(i, attn_only)
                ones.append(g1)
            self.g_one[attn_only] = ones
        torch.cuda.synchronize()

    def _step(self, i, attention_only=False):
        p = self.paths[i]
        if self.fused:
            p.step_fused()          # the step is the attention call
        elif attention_only:
            p.attention()
        else:
            p.step()

    def run(self, n, attention_only=False):
        """Exactly n steps, cycling over the copies."""
        n_copies = len(self.paths)
        if not self.use_graph:
            for i in range(n):
                self._step(i % n_copies, attention_only)
            return
        whole, rest = divmod(n, n_copies)
        for _ in range(whole):
            self.g_all[attention_only].replay()
        for i in range(rest):
            self.g_one[attention_only][i].replay()


def rotate_copies(wl, requested):
    if requested > 0:
        return requested
    bytes_attn, _, _ = algorithmic_cost(wl)
    return max(2, -(-ROTATE_BYTES // max(1, bytes_attn)))


def time_attention(name, wl, args, stream, steps, warmup, min_sample_ms):
    """Upload ``copies`` of the batch, prepare their context keys, and time
    (a) exactly ``steps`` steps between synchronisations (the step time), and
    (b) the attention call alone with HIP events on its stream over at least
    ``min_sample_ms`` (the dominant kernel's average launch time)."""
    import torch
    from block_diffusion_draft_dflash_amd.pipeline import DevicePath

    copies = rotate_copies(wl, args.rotate)
    paths = [DevicePath(wl, split_keys=args.split_keys, host_lengths=not args.device_plan,
                        paged=args.paged) for _ in range(copies)]
    for p in paths:
        p.prepare_context()
    torch.cuda.synchronize()
    fused = wl.dtype == "bf16" and not args.unfused
    use_graph = not args.no_graph
    runner = StepRunner(paths, fused, use_graph)

    runner.run(warmup)
    torch.cuda.synchronize()
    # ---- timed region: exactly `steps` steps
    t0 = time.perf_counter()
    runner.run(steps)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / max(steps, 1)

    # ---- the attention call alone, HIP events on its stream
    est_us = max(ms_per_step * 1e3, 1.0)
    n_attn = max(steps, int(math.ceil(min_sample_ms * 1e3 / est_us)))
    n_attn = -(-n_attn // copies) * copies
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    runner.run(n_attn, attention_only=True)
    ev1.record(stream)
    torch.cuda.synchronize()
    attn_us = ev0.elapsed_time(ev1) * 1e3 / n_attn

    bytes_attn, flops_attn, bytes_pro = algorithmic_cost(wl)
    achieved = bytes_attn / (attn_us * 1e-6) / 1e9
    rec = {
        "workload": name, "requests": wl.num_reqs, "context_rows": wl.total_ctx,
        "block_rows": wl.total_blk, "hq": wl.hq, "hkv": wl.hkv, "dh": wl.dh,
        "mask": ("causal, window %d" % wl.window) if wl.causal else "bidirectional",
        "rotating_copies": copies, "steps": steps, "warmup": warmup,
        "ms_per_step": ms_per_step,
        "tflops": flops_attn / (ms_per_step * 1e-3) / 1e12,
        "draft_query_tokens_per_s": wl.total_blk / (ms_per_step * 1e-3),
        "attention_call_us": attn_us, "attention_calls_timed": n_attn,
        "achieved_gbs": achieved, "frac_of_hbm_peak": achieved / HBM_PEAK_GBS,
        "attention_bytes": bytes_attn, "attention_flops": flops_attn,
        "prologue_bytes": bytes_pro, "fused": fused, "hip_graph": use_graph,
    }
    return rec, paths


def time_context_kv(wl, path, stream, reps=5):
    """The dflash_context_kv call (weight fold, fused GEMM + row rms + k-norm +
    RoPE) with HIP events on its stream, against the dense bf16 MFMA peak, and
    one whole pass of precompute then the attention step."""
    import torch
    path.prepare_context()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        path.prepare_context()
    e1.record(stream)
    torch.cuda.synchronize()
    ckv_ms = e0.elapsed_time(e1) / reps
    flops = 2.0 * wl.total_ctx * wl.hidden_size * (2 * wl.hkv * wl.dh)
    tflops = flops / (ckv_ms * 1e-3) / 1e12
    # algorithmic bytes: hidden rows in, weights in, K and V caches out
    bytes_ckv = (wl.total_ctx * wl.hidden_size * 2 + 2 * wl.hkv * wl.dh * wl.hidden_size * 2
                 + 2 * wl.total_ctx * wl.hkv * wl.dh * 2)
    e0.record(stream)
    for _ in range(reps):
        path.prepare_context()
        path.step_fused()
    e1.record(stream)
    torch.cuda.synchronize()
    pass_ms = e0.elapsed_time(e1) / reps
    return (
        {"ms": ckv_ms, "tflops": tflops, "bound": "mfma", "peak_tflops": BF16_PEAK_TFLOPS,
         "frac": tflops / BF16_PEAK_TFLOPS, "flops": flops, "bytes": bytes_ckv,
         "rows": wl.total_ctx, "hidden": wl.hidden_size, "calls_timed": reps},
        {"ms": pass_ms, "stages": "dflash_context_kv then dflash_block_attention (fused)",
         "passes_timed": reps},
    )


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
        "hidden": hidden, "weight_copies": copies, "block_rows": t,
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
    block q/k/v, the paged attention (work split planned on the device, the
    batch's mask flags) and o_proj. Each request verifies one block of rows on
    top of its context."""
    import torch
    from block_diffusion_draft_dflash_amd.pipeline import DraftStep

    nqpr = int(wl.blk_lens.max())
    rows = nqpr
    pages = (int(wl.ctx_lens.max()) + rows + 15) // 16 + 1
    ds = DraftStep(wl.num_reqs, nqpr, rows, hidden=hidden, taps=taps, hq=wl.hq, hkv=wl.hkv,
                   dh=wl.dh, pages_per_req=pages, seed=11, causal=wl.causal, window=wl.window)
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
    ap.add_argument("--steps", type=int, default=600)
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--workload", default="ctx_kv")
    ap.add_argument("--rotate", type=int, default=0,
                    help="copies of the batch cycled per step (0: enough to span 512 MiB)")
    ap.add_argument("--min-sample-ms", type=float, default=30.0,
                    help="GPU time the attention-call timing (HIP events) spans at least")
    ap.add_argument("--split-keys", type=int, default=0)
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    ap.add_argument("--unfused", action="store_true",
                    help="q/k norm + RoPE as a separate in-place call before the attention")
    ap.add_argument("--paged", action="store_true",
                    help="read the context from a paged store (dflash_block_attention_paged)")
    ap.add_argument("--device-plan", action="store_true",
                    help="leave the work split to the kernels (no host copies of the lengths)")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle time (0: skip)")
    ap.add_argument("--sub-configs", default=",".join(SUB_CONFIGS),
                    help="other workloads timed in the same run as sub-records ('' for none)")
    ap.add_argument("--layer-hidden", type=int, default=4096,
                    help="hidden size of the draft layer whose projections around the attention "
                         "(dflash_block_qkv, dflash_o_proj) are also timed (0: skip)")
    ap.add_argument("--layer-workload", default="qwen3_8b_draft",
                    help="the batch the draft layer and the propose step are timed on")
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
    if args.steps < 1 or args.warmup < 0:
        print("bench.py: --steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import torch
    from block_diffusion_draft_dflash_amd import binding as B
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
    stream = torch.cuda.current_stream()

    wl = make_workload(args.workload)
    head, paths = time_attention(args.workload, wl, args, stream, args.steps, args.warmup,
                                 args.min_sample_ms)

    ckv = full_pass = None
    if wl.hidden is not None:
        ckv, full_pass = time_context_kv(wl, paths[0], stream)
    del paths
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    # the dominant kernel's traffic, from the committed counter record: only
    # for the default launch (packed store, fused prologue, host-planned split)
    default_launch = not (args.paged or args.unfused or args.device_plan or args.split_keys)
    traffic = committed_traffic(args.workload) if default_launch else None
    copy_gbs = device_copy_gbs(stream) if args.copy_calibration_mb == 0 else None

    subs = {}
    for name in [s for s in args.sub_configs.split(",") if s and s != args.workload]:
        swl = make_workload(name)
        if swl.dtype != "bf16":
            continue
        rec, spaths = time_attention(name, swl, args, stream, max(args.steps, 120),
                                     max(args.warmup, 12), args.min_sample_ms)
        rec["traffic"] = committed_traffic(name) if default_launch else None
        subs[name] = rec
        del spaths
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

    layer = draft_step = None
    if args.layer_hidden > 0 and not args.paged:
        lwl = wl if args.layer_workload == args.workload else make_workload(args.layer_workload)
        if lwl.dtype == "bf16":
            layer = time_layer(lwl, args.layer_hidden, stream, not args.no_graph)
            layer["workload"] = args.layer_workload
            torch.cuda.empty_cache()
            if args.draft_step_taps > 0:
                draft_step = time_draft_step(lwl, args.layer_hidden, args.draft_step_taps, stream)
                draft_step["workload"] = args.layer_workload

    cpu = None
    if args.cpu_budget > 0:
        cb = cpu_baseline(wl, args.cpu_budget, ctx_rows=None)
        cpu = {
            "value": cb["flops"] / cb["seconds"] / 1e12,
            "unit": "TFLOP/s",
            "cores": cb["threads"],
            "kind": "oracle",
            "sample": (f"fp64 numpy oracle on {cb['sample']}; {cb['passes']} passes in "
                       f"{cb['seconds'] * cb['passes']:.1f} s"),
            "ms_per_step": cb["seconds"] * 1e3,
            "draft_query_tokens_per_s": cb["query_rows"] / cb["seconds"],
            "cpu_model": cb["cpu_model"],
            "cores_available": cb["cores_available"],
        }
        if cb["context_kv"] is not None:
            c = cb["context_kv"]
            cpu["context_kv"] = {"rows": c["rows"], "seconds": c["seconds"],
                                 "tflops": c["flops"] / c["seconds"] / 1e12}

    bytes_attn = head["attention_bytes"]
    rec = {
        "metric": "block-attention TFLOP/s and draft query tokens/s; % of MI355X roofline",
        "value": head["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
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
            "hidden": wl.hidden_size or None,
            "mask": head["mask"],
            "rotating_copies": head["rotating_copies"],
            "hip_graph": head["hip_graph"],
            "fused_qk_norm_rope": head["fused"],
            "work_split": "device-planned" if args.device_plan else "host-planned",
            "context_store": "paged (16-row pages)" if args.paged else "packed",
        },
        "draft_query_tokens_per_s": head["draft_query_tokens_per_s"],
        "roofline": {
            "bound": "hbm",
            "kernel": ("dflash_block_attention%s call = block_attn_bf16_kernel%s + "
                       "block_attn_merge_kernel" % ("_paged" if args.paged else "",
                                                    " (fused q/k norm + RoPE)" if head["fused"] else "")),
            "achieved": head["achieved_gbs"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": head["frac_of_hbm_peak"],
            "traffic": traffic,
            "algorithmic_bytes_per_launch": bytes_attn,
            "avg_launch_us": head["attention_call_us"],
            "launches_timed": head["attention_calls_timed"],
            "achievable_copy_gbs": copy_gbs,
            "frac_of_copy": head["achieved_gbs"] / copy_gbs if copy_gbs else None,
        },
        "cpu_baseline": cpu,
        "context_kv": ckv,
        "full_pass": full_pass,
        "configs": subs,
        "draft_layer": layer,
        "draft_step": draft_step,
        "algorithmic": {"attention_bytes": bytes_attn, "attention_flops": head["attention_flops"],
                        "prologue_bytes": head["prologue_bytes"]},
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
