"""Host-side logic of bench.py (CPU only): the oracle's timed sample on every
kind of workload, the exact step count of the graph runner, the rotation
count, and the algorithmic cost of a batch."""
import numpy as np

import bench
from block_diffusion_draft_dflash_amd.workloads import make_workload


def test_cpu_baseline_hidden_state_workload():
    # a workload given as hidden states: the oracle builds its own context K/V
    wl = make_workload("ctx_kv", num_reqs=2, ctx_len=40, hidden=64)
    cb = bench.cpu_baseline(wl, 0.01)
    assert cb["passes"] >= 1 and cb["seconds"] > 0
    assert cb["context_kv"]["rows"] == 40
    # request 0's 16 block rows over its 40 context rows + 16 block rows
    assert cb["flops"] == 16 * 56 * wl.hq * 4 * wl.dh
    assert cb["query_rows"] == 16
    assert cb["threads"] >= 1 and cb["cores_available"] >= 1 and cb["cpu_model"]


def test_cpu_baseline_key_workloads():
    wl = make_workload("qwen3_8b_draft", num_reqs=3, ctx_lo=20, ctx_hi=60)
    cb = bench.cpu_baseline(wl, 0.01)
    _, flops, _ = bench.algorithmic_cost(wl)
    assert cb["flops"] == flops and cb["context_kv"] is None
    sw = make_workload("swa", num_reqs=3, ctx_len=50, window=20)
    cb = bench.cpu_baseline(sw, 0.01, sample_reqs=2)
    # causal + window: each query sees min(window, its index + 1) keys
    per_req = sum(min(20, 50 + i + 1) for i in range(16))
    assert cb["flops"] == 2 * per_req * sw.hq * 4 * sw.dh


class _CountingPath:
    def __init__(self):
        self.calls = 0

    def step_fused(self):
        self.calls += 1


def test_step_runner_runs_exactly_the_requested_steps():
    paths = [_CountingPath() for _ in range(3)]
    r = bench.StepRunner(paths, fused=True, use_graph=False)
    for n in (0, 1, 5, 20):
        before = sum(p.calls for p in paths)
        r.run(n)
        assert sum(p.calls for p in paths) - before == n


def test_rotation_spans_the_cache():
    for name in ("qwen3_8b_draft", "large_decode"):
        wl = make_workload(name, num_reqs=4)
        b, _, _ = bench.algorithmic_cost(wl)
        n = bench.rotate_copies(wl, 0)
        assert n >= 2 and n * b >= bench.ROTATE_BYTES
    assert bench.rotate_copies(wl, 5) == 5


def test_algorithmic_cost_counts_visible_keys():
    wl = make_workload("swa", num_reqs=2, ctx_len=100, window=30)
    b, f, p = bench.algorithmic_cost(wl)
    kv_row = 2 * wl.hkv * wl.dh * 2
    vis = 2 * (100 + 16 - (100 - 30 + 1))
    assert b == vis * kv_row + 2 * 2 * 16 * wl.hq * wl.dh * 2
    assert p == 2 * 32 * (wl.hq + wl.hkv) * wl.dh * 2
    assert np.all(wl.visible_keys() == 100 + 16 - 71)
