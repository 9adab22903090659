"""The allocation-free entry point (dflash_block_attention_noalloc, for
callers that cannot allocate) against dflash_block_attention with a caller
workspace: two calls in a row on the same GPU, the second on a smaller batch
(the scratch then holds the first call's partials), each bitwise equal to the
workspace call on the same inputs and within the bf16 output bars of the
fp64 oracle. Then the same call captured into a HIP graph and replayed."""
import numpy as np
import pytest
import torch

from block_diffusion_draft_dflash_amd import binding as B
from block_diffusion_draft_dflash_amd.pipeline import DevicePath, to_host_f64
from block_diffusion_draft_dflash_amd.workloads import make_workload

pytestmark = pytest.mark.gpu


def _oracle(wl):
    from oracle import dflash_oracle as O
    _, k_ctx = O.qk_norm_rope(None, wl.k_ctx, None, wl.k_norm_w, wl.ctx_positions, wl.eps, wl.theta)
    out, _, _ = O.draft_block_attention(wl.q, wl.k_blk, wl.v_blk, wl.blk_positions, k_ctx, wl.v_ctx,
                                        wl.cu_ctx, wl.cu_blk, wl.q_norm_w, wl.k_norm_w, wl.eps,
                                        wl.theta, wl.scale, wl.causal, wl.window)
    return out


def _noalloc(dp, out, fused):
    q, kb = (dp.q_raw, dp.k_blk_raw) if fused else (dp.q, dp.k_blk)
    B.dflash_block_attention_noalloc(dp.params, dp.cu_ctx, dp.cu_blk, q, kb, dp.v_blk, dp.k_ctx,
                                     dp.v_ctx, out, prologue=dp.prologue if fused else None)


CASES = [
    # (workload, overrides, oracle check): the first needs 17 MiB of scratch
    ("large_decode", dict(num_reqs=64, ctx_lo=128, ctx_hi=8192), False),
    ("qwen3_8b_draft", dict(num_reqs=3, ctx_lo=100, ctx_hi=700), True),
]


@pytest.mark.parametrize("fused", [True, False])
def test_noalloc_matches_the_workspace_call(dflash, fused):
    for name, kw, with_oracle in CASES:
        print(f"case noalloc {name} {kw} fused={fused}", flush=True)
        wl = make_workload(name, **kw)
        dp = DevicePath(wl)
        assert B.dflash_block_attention_workspace_size(dp.params) <= B.NOALLOC_SCRATCH_BYTES
        dp.prepare_context()
        if not fused:
            dp.qk_norm_rope()
        (dp.attention_fused if fused else dp.attention)()
        torch.cuda.synchronize()
        ref = dp.out.clone()
        got = torch.full_like(dp.out, float("nan"))
        _noalloc(dp, got, fused)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"{name}: not bitwise equal"
        if with_oracle:
            err = np.abs(to_host_f64(got) - _oracle(wl))
            print(f"[noalloc {name}] max abs {err.max():.3e} mean abs {err.mean():.3e}", flush=True)
            assert err.max() <= 2e-2 and err.mean() <= 2e-3


def test_noalloc_graph_replay(dflash):
    print("case noalloc graph replay", flush=True)
    wl = make_workload("qwen3_8b_draft", num_reqs=4, ctx_lo=200, ctx_hi=900)
    dp = DevicePath(wl)
    dp.prepare_context()
    dp.attention_fused()
    torch.cuda.synchronize()
    ref = dp.out.clone()
    got = torch.zeros_like(dp.out)
    _noalloc(dp, got, True)          # first call on the device: address lookup, outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _noalloc(dp, got, True)
    scratch = torch.randn(1 << 20, device="cuda")
    for i in range(3):
        got.fill_(float("nan"))
        scratch.mul_(1.0001)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"replay {i}"
