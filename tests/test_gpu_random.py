"""Seeded random batches through the whole attention path, each against the
fp64 oracle (the bars of test_gpu_parity.py).

Every case draws its own combination of what the other tests vary one at a
time: request count, ragged context lengths (empty ones included), block
lengths up to the fused prologue's 64 rows (empty ones included), GQA group
and kv-head count, head dim, bidirectional / causal / causal with a window
(shorter or longer than the rows), forced or planned splits, host or device
planning, packed or paged context store, fused prologue or the standalone
norm + RoPE, bf16 or f32. The draws are fixed by the case number.
"""
import os

import numpy as np
import pytest
import torch

from block_diffusion_draft_dflash_amd.pipeline import DevicePath
from block_diffusion_draft_dflash_amd.workloads import make_workload
from test_gpu_parity import assert_output, gpu_rows, oracle_outputs

pytestmark = pytest.mark.gpu

# 64 cases by default; DFLASH_RANDOM_CASES=N runs the first N seeds
N_CASES = int(os.environ.get("DFLASH_RANDOM_CASES", "64"))


def draw(i):
    rng = np.random.default_rng(7100 + i)
    f32 = i % 8 == 7
    r = int(rng.integers(1, 11))
    ctx = rng.integers(0, 901, r) * (rng.random(r) > 0.15)
    blk = rng.integers(1, 65, r) * (rng.random(r) > 0.15)
    if blk.sum() == 0:
        blk[0] = int(rng.integers(1, 65))
    hkv = int(rng.choice([1, 2, 4, 8]))
    group = int(rng.choice([1, 2, 4, 8, 16]))
    dh = int(rng.choice([64, 128]))
    mode = rng.choice(["bidirectional", "causal", "window"])
    causal = mode != "bidirectional"
    window = int(rng.integers(1, 1200)) if mode == "window" else 0
    split = int(rng.choice([0, 0, 0, 64, 128, 320, 4096]))
    host = bool(rng.random() < 0.6)
    paged = bool(rng.random() < 0.25)
    fused = (not f32) and bool(rng.random() < 0.5)
    over = dict(ctx_lens=ctx.tolist(), blk_lens=blk.tolist(), hq=hkv * group, hkv=hkv, dh=dh,
                causal=causal, window=window)
    if f32:
        over["dtype"] = "f32"
    return over, dict(split_keys=split, host_lengths=host, paged=paged), fused


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_batch(i):
    over, path_kw, fused = draw(i)
    tag = (f"random {i}: R={len(over['ctx_lens'])} Hq={over['hq']} Hkv={over['hkv']} Dh={over['dh']} "
           f"causal={over['causal']} window={over['window']} {path_kw} fused={fused} "
           f"{over.get('dtype', 'bf16')}")
    print("case", tag, flush=True)
    wl = make_workload("qwen3_8b_draft", seed=7100 + i, **over)
    dp = DevicePath(wl, **path_kw)
    dp.prepare_context()
    if fused:
        dp.step_fused()
    else:
        dp.step()
    torch.cuda.synchronize()
    ref = oracle_outputs(wl)
    reqs = list(range(wl.num_reqs))
    assert_output(wl, gpu_rows(wl, dp.out, reqs), ref["out"], tag)
