"""Paged context store on the GPU: dflash_kv_scatter and dflash_block_attention_paged.

The paged call reads the context rows through a block table of 16-row pages
handed out in a random order over a NaN-filled pool (spare pages unused), so
a read of any slot the table does not map would surface as NaN. With the
same split as the packed call its output must be bitwise the packed call's
(which the parity tests hold to the oracle).
"""
import numpy as np
import pytest
import torch

from block_diffusion_draft_dflash_amd.pipeline import DevicePath
from block_diffusion_draft_dflash_amd.workloads import make_workload

pytestmark = pytest.mark.gpu

CASES = {
    "qwen3_8b_draft_small": dict(name="qwen3_8b_draft", num_reqs=3, ctx_lo=100, ctx_hi=700),
    "swa_unaligned_window": dict(name="swa", num_reqs=3, ctx_len=700, window=203),
    "large_decode_70req": dict(name="large_decode", num_reqs=70, ctx_lo=1, ctx_hi=300),
    "empty_ctx_and_blocks": dict(name="qwen3_8b_draft", ctx_lens=[0, 5, 130, 0, 77],
                                 blk_lens=[3, 0, 17, 40, 1]),
    "dh64": dict(name="qwen3_8b_draft", num_reqs=3, ctx_lo=50, ctx_hi=300, hq=8, hkv=2, dh=64),
    "gqa8": dict(name="qwen3_8b_draft", num_reqs=2, ctx_lo=50, ctx_hi=200, hq=64, hkv=8),
    "ctx_kv_hidden": dict(name="ctx_kv", num_reqs=2, ctx_len=300, hidden=512),
    "f32_tiny": dict(name="tiny", ctx_lens=[64, 129, 0], blk_lens=[16, 5, 7]),
}


def _pair(case, host_lengths):
    kw = dict(CASES[case])
    name = kw.pop("name")
    wl = make_workload(name, **kw)
    packed = DevicePath(wl, host_lengths=host_lengths)
    paged = DevicePath(wl, host_lengths=host_lengths, paged=True)
    packed.prepare_context()
    paged.prepare_context()
    return wl, packed, paged


@pytest.mark.parametrize("host_lengths", [True, False])
@pytest.mark.parametrize("case", list(CASES))
def test_paged_bitwise_equals_packed(case, host_lengths):
    print(f"case paged {case} host_lengths={host_lengths}", flush=True)
    wl, packed, paged = _pair(case, host_lengths)
    bits = (lambda t: t.view(torch.int16)) if wl.dtype == "bf16" else (lambda t: t.view(torch.int32))
    steps = ["step_fused", "step"] if wl.dtype == "bf16" else ["step"]
    for how in steps:  # the fused call first: step() normalises q and k in place
        getattr(packed, how)()
        getattr(paged, how)()
        torch.cuda.synchronize()
        assert not torch.isnan(paged.out.float()).any(), f"{how}: NaN (an unmapped slot was read)"
        assert torch.equal(bits(paged.out), bits(packed.out)), f"{how}: paged != packed"


def test_paged_full_qwen3_8b_draft():
    print("case paged full qwen3_8b_draft", flush=True)
    wl = make_workload("qwen3_8b_draft")
    packed = DevicePath(wl)
    paged = DevicePath(wl, paged=True)
    packed.prepare_context()
    paged.prepare_context()
    packed.step_fused()
    paged.step_fused()
    torch.cuda.synchronize()
    assert torch.equal(paged.out.view(torch.int16), packed.out.view(torch.int16))


def test_kv_scatter(dflash):
    print("case kv_scatter", flush=True)
    g = torch.Generator(device="cpu").manual_seed(7)
    t, hkv, dh, nslots = 300, 8, 128, 1000
    k = torch.randn(t, hkv, dh, generator=g).to(torch.bfloat16).cuda()
    v = torch.randn(t, hkv, dh, generator=g).to(torch.bfloat16).cuda()
    slots = torch.randperm(nslots, generator=g)[:t].to(torch.int32)
    slots[::17] = -1           # padding rows are skipped
    slots[5] = nslots + 3      # so is a slot past the pool
    kp = torch.full((nslots // 16 * 16 // 16, 16, hkv, dh), float("nan"), dtype=torch.bfloat16).cuda()
    vp = torch.full_like(kp, float("nan"))
    dflash.dflash_kv_scatter(k, v, slots.cuda(), kp, vp)
    torch.cuda.synchronize()
    kf, vf = kp.view(-1, hkv, dh).cpu(), vp.view(-1, hkv, dh).cpu()
    valid = (slots >= 0) & (slots < kf.shape[0])
    idx = slots[valid].long()
    assert torch.equal(kf[idx].view(torch.int16), k.cpu()[valid].view(torch.int16))
    assert torch.equal(vf[idx].view(torch.int16), v.cpu()[valid].view(torch.int16))
    untouched = torch.ones(kf.shape[0], dtype=torch.bool)
    untouched[idx] = False
    assert torch.isnan(kf[untouched].float()).all() and torch.isnan(vf[untouched].float()).all()


def test_paged_unit_cap(dflash):
    # With 64 kv-heads and one request the packed call plans 4 units per
    # head (one per compute unit), so the 140000 context rows go in splits of
    # about 35000 keys; over a paged store units are capped at 16384 keys
    # (more units, other rounding).
    print("case paged unit cap", flush=True)
    torch.manual_seed(11)
    hq = hkv = 64
    dh = 64
    c, b = 140000, 16
    dev = "cuda"
    kc = torch.randn(c, hkv, dh, device=dev).to(torch.bfloat16)
    vc = torch.randn(c, hkv, dh, device=dev).to(torch.bfloat16)
    q = torch.randn(b, hq, dh, device=dev).to(torch.bfloat16)
    kb = torch.randn(b, hkv, dh, device=dev).to(torch.bfloat16)
    vb = torch.randn(b, hkv, dh, device=dev).to(torch.bfloat16)
    cu_c = torch.tensor([0, c], dtype=torch.int32, device=dev)
    cu_b = torch.tensor([0, b], dtype=torch.int32, device=dev)
    p = dflash.make_block_attn_params(1, hq, hkv, dh, dflash.DFLASH_BF16, c, b, b, dh ** -0.5)
    npages = (c + 15) // 16
    perm = torch.randperm(npages + 3, generator=torch.Generator().manual_seed(3))[:npages]
    bt = perm.to(torch.int32).view(1, -1).to(dev)
    slots = (bt.view(-1).long().repeat_interleave(16)[:c] * 16 +
             torch.arange(c, device=dev) % 16).to(torch.int32)
    kp = torch.full((npages + 3, 16, hkv, dh), float("nan"), dtype=torch.bfloat16, device=dev)
    vp = torch.full_like(kp, float("nan"))
    dflash.dflash_kv_scatter(kc, vc, slots, kp, vp)
    pg = dflash.make_paged_ctx(bt, npages + 3)
    out_packed = torch.empty_like(q)
    out_paged = torch.empty_like(q)
    ws1 = dflash.alloc_workspace(dflash.dflash_block_attention_workspace_size(p))
    ws2 = dflash.alloc_workspace(dflash.dflash_block_attention_paged_workspace_size(p))
    dflash.dflash_block_attention(p, cu_c, cu_b, q, kb, vb, kc, vc, out_packed, ws1)
    dflash.dflash_block_attention_paged(p, pg, cu_c, cu_b, q, kb, vb, kp, vp, out_paged, ws2)
    torch.cuda.synchronize()
    d = (out_paged.float() - out_packed.float()).abs()
    print(f"[paged unit cap] max abs diff {d.max().item():.3e} mean {d.mean().item():.3e}")
    assert not torch.isnan(out_paged.float()).any()
    assert d.max().item() <= 2e-2 and d.mean().item() <= 2e-3


@pytest.mark.parametrize("case", ["swa_unaligned_window", "empty_ctx_and_blocks"])
def test_paged_vs_oracle_through_the_pools(case):
    # the oracle reads the context rows out of the device pools by the paged
    # layout's definition and computes the attention on them
    from block_diffusion_draft_dflash_amd.pipeline import to_host_f64
    from oracle import dflash_oracle as O
    print(f"case paged oracle {case}", flush=True)
    kw = dict(CASES[case])
    name = kw.pop("name")
    wl = make_workload(name, **kw)
    dp = DevicePath(wl, paged=True)
    dp.prepare_context()
    dp.step_fused()
    torch.cuda.synchronize()
    bt = dp.block_table.cpu().numpy()
    k_ctx = O.paged_context_rows(to_host_f64(dp.k_pool), bt, wl.ctx_lens)
    v_ctx = O.paged_context_rows(to_host_f64(dp.v_pool), bt, wl.ctx_lens)
    ref, _, _ = O.draft_block_attention(wl.q, wl.k_blk, wl.v_blk, wl.blk_positions, k_ctx, v_ctx,
                                        wl.cu_ctx, wl.cu_blk, wl.q_norm_w, wl.k_norm_w, wl.eps,
                                        wl.theta, wl.scale, wl.causal, wl.window)
    err = np.abs(to_host_f64(dp.out) - ref)
    print(f"[paged oracle {case}] max abs {err.max():.3e} mean abs {err.mean():.3e}")
    assert err.max() <= 2e-2 and err.mean() <= 2e-3
    # and independently of the pools: the oracle's own context rows (its norm
    # + RoPE of the raw keys, the raw values) against what the pools hold
    # through the block table, and the attention on the oracle's rows
    _, k_own = O.qk_norm_rope(None, wl.k_ctx, None, wl.k_norm_w, wl.ctx_positions, wl.eps, wl.theta)
    bad = np.abs(k_ctx - k_own) > 2.0 ** -7 * np.abs(k_own) + 1e-5
    assert not bad.any(), f"{bad.sum()} pooled K elements beyond one rounding of the oracle's"
    assert np.array_equal(v_ctx, np.asarray(wl.v_ctx, dtype=np.float64)), "pooled V differs from the input"
    ref_own, _, _ = O.draft_block_attention(wl.q, wl.k_blk, wl.v_blk, wl.blk_positions, k_own,
                                            wl.v_ctx, wl.cu_ctx, wl.cu_blk, wl.q_norm_w, wl.k_norm_w,
                                            wl.eps, wl.theta, wl.scale, wl.causal, wl.window)
    err = np.abs(to_host_f64(dp.out) - ref_own)
    print(f"[paged oracle {case}, oracle's own context rows] max abs {err.max():.3e} mean abs {err.mean():.3e}")
    assert err.max() <= 2e-2 and err.mean() <= 2e-3
