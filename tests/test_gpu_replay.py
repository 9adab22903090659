"""Repeat, planning and graph-replay behaviour of dflash_block_attention on the GPU.

  * repeated calls on one workspace give bitwise the same output;
  * the work split planned on the host (host copies of the lengths given)
    and the one the kernels plan from the device arrays are the same plan:
    bitwise the same output;
  * a HIP graph of the call replays to the eager result, replay after replay,
    with other device work and host synchronisation between the replays.
"""
import pytest
import torch

from block_diffusion_draft_dflash_amd.pipeline import DevicePath
from block_diffusion_draft_dflash_amd.workloads import make_workload

pytestmark = pytest.mark.gpu

CASES = {
    "qwen3_8b_draft": dict(name="qwen3_8b_draft"),
    "large_decode_small": dict(name="large_decode", num_reqs=70, ctx_lo=1, ctx_hi=300),
    "swa_small": dict(name="swa", num_reqs=3, ctx_len=700, window=256),
    "split64": dict(name="qwen3_8b_draft", num_reqs=3, ctx_lo=100, ctx_hi=700, split_keys=64),
}


def _path(case, host_lengths=True):
    kw = dict(CASES[case])
    name = kw.pop("name")
    split = kw.pop("split_keys", 0)
    wl = make_workload(name, **kw)
    dp = DevicePath(wl, split_keys=split, host_lengths=host_lengths)
    dp.prepare_context()
    return wl, dp


@pytest.mark.parametrize("host_lengths", [True, False])
@pytest.mark.parametrize("case", list(CASES))
def test_repeat_bitwise(case, host_lengths):
    print(f"case repeat {case} host_lengths={host_lengths}", flush=True)
    wl, dp = _path(case, host_lengths)
    outs = []
    for _ in range(3):
        dp.out.zero_()
        dp.step_fused()
        torch.cuda.synchronize()
        outs.append(dp.out.clone())
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))


@pytest.mark.parametrize("case", list(CASES))
def test_host_and_device_plans_agree(case):
    print(f"case plans {case}", flush=True)
    _, dh = _path(case, True)
    _, dd = _path(case, False)
    dh.step_fused()
    dd.step_fused()
    torch.cuda.synchronize()
    assert torch.equal(dh.out.view(torch.int16), dd.out.view(torch.int16)), "fused"
    dh.step()  # unfused: in-place norm + RoPE (once), then attention on the normed rows
    dd.step()
    torch.cuda.synchronize()
    assert torch.equal(dh.out.view(torch.int16), dd.out.view(torch.int16)), "unfused"


@pytest.mark.parametrize("host_lengths", [True, False])
@pytest.mark.parametrize("case", ["qwen3_8b_draft", "large_decode_small"])
def test_graph_replay_matches_eager(case, host_lengths):
    print(f"case graph {case} host_lengths={host_lengths}", flush=True)
    wl, dp = _path(case, host_lengths)
    dp.step_fused()
    torch.cuda.synchronize()
    ref = dp.out.clone()
    dp.step_fused()  # warm the launch path before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dp.step_fused()
        dp.step_fused()
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device=dp.out.device)
    for i in range(4):
        dp.out.zero_()
        scratch.mul_(1.0001).add_(0.5)  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dp.out.view(torch.int16), ref.view(torch.int16)), f"replay {i} differs"
