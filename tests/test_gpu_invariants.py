"""GPU invariants of the block attention that hold whatever the oracle says:

  * a packed varlen batch equals each request launched alone, bitwise, when
    the keys are cut at the same boundaries (a fixed split size);
  * the f32 path and the bf16 path agree, on inputs that are exactly
    bf16-representable, within the bf16 output bars (max abs 2e-2, mean abs
    2e-3).
"""
import dataclasses

import numpy as np
import pytest
import torch

from block_diffusion_draft_dflash_amd.pipeline import DevicePath, to_host_f64
from block_diffusion_draft_dflash_amd.workloads import make_workload

pytestmark = pytest.mark.gpu


def one_request(wl, r):
    """The workload restricted to request r (context and block rows re-based)."""
    c0, c1 = int(wl.cu_ctx[r]), int(wl.cu_ctx[r + 1])
    b0, b1 = int(wl.cu_blk[r]), int(wl.cu_blk[r + 1])
    i32 = lambda *v: np.asarray(v, dtype=np.int32)
    return dataclasses.replace(
        wl, num_reqs=1, ctx_lens=wl.ctx_lens[r:r + 1], blk_lens=wl.blk_lens[r:r + 1],
        cu_ctx=i32(0, c1 - c0), cu_blk=i32(0, b1 - b0),
        ctx_positions=wl.ctx_positions[c0:c1], blk_positions=wl.blk_positions[b0:b1],
        q=wl.q[b0:b1], k_blk=wl.k_blk[b0:b1], v_blk=wl.v_blk[b0:b1],
        k_ctx=wl.k_ctx[c0:c1], v_ctx=wl.v_ctx[c0:c1])


def run(wl, fused, split_keys=0, host_lengths=True):
    dp = DevicePath(wl, split_keys=split_keys, host_lengths=host_lengths)
    dp.prepare_context()
    if fused:
        dp.step_fused()
    else:
        dp.step()
    torch.cuda.synchronize()
    return dp.out.clone()


CASES = {
    "qwen3_8b_draft": dict(name="qwen3_8b_draft", num_reqs=5, ctx_lo=60, ctx_hi=900),
    "swa": dict(name="swa", num_reqs=3, ctx_len=500, window=200),
    "ragged": dict(name="qwen3_8b_draft", ctx_lens=[0, 5, 130, 0, 77], blk_lens=[3, 0, 17, 40, 1]),
}


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("case", list(CASES))
def test_varlen_batch_equals_each_request_alone(case, fused):
    print(f"case varlen vs per-request {case} fused={fused}", flush=True)
    kw = dict(CASES[case])
    wl = make_workload(kw.pop("name"), **kw)
    split = 128  # the same key boundaries in the batch and alone
    whole = run(wl, fused, split_keys=split)
    for r in range(wl.num_reqs):
        b0, b1 = int(wl.cu_blk[r]), int(wl.cu_blk[r + 1])
        if b1 == b0:
            continue
        alone = run(one_request(wl, r), fused, split_keys=split)
        assert torch.equal(whole[b0:b1], alone), f"request {r}: batch != alone"
        # and planned on the device instead of the host: the same bits
        dev = run(one_request(wl, r), fused, split_keys=split, host_lengths=False)
        assert torch.equal(alone, dev), f"request {r}: device plan != host plan"


@pytest.mark.parametrize("case", ["qwen3_8b_draft", "swa", "ragged"])
def test_f32_and_bf16_paths_agree(case):
    print(f"case f32 vs bf16 {case}", flush=True)
    kw = dict(CASES[case])
    wl = make_workload(kw.pop("name"), **kw)
    got16 = to_host_f64(run(wl, fused=False))
    got32 = to_host_f64(run(dataclasses.replace(wl, dtype="f32"), fused=False))
    err = np.abs(got16 - got32)
    print(f"[{case}] max abs {err.max():.3e} mean abs {err.mean():.3e}", flush=True)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3
