"""The DFLASH_VALIDATE debug mode on the GPU.

With the variable set, the calls that take integer metadata on the device copy
it to the host first and refuse, before enqueueing anything, what breaks the
preconditions the "qwen3_dflash.cpp" page checks on the host (ForwardWithCtxKVDev
and ForwardPagedBody: cumulative lengths starting at 0 and spanning the rows;
PrecomputeContextKVDevice: positions; the paged store's block table): every
rejected call here launches no kernel. Valid batches give the same bits as
without the mode, and a stream that is being captured is refused.
"""
import pytest
import torch

from block_diffusion_draft_dflash_amd import binding as B
from block_diffusion_draft_dflash_amd.pipeline import DevicePath
from block_diffusion_draft_dflash_amd.workloads import make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture
def validate(monkeypatch):
    monkeypatch.setenv("DFLASH_VALIDATE", "1")


def small(**kw):
    return make_workload("qwen3_8b_draft", num_reqs=3, ctx_lo=100, ctx_hi=300, **kw)


def rejected(fn, status, text):
    with pytest.raises(B.DflashError) as ei:
        fn()
    msg = str(ei.value)
    print("rejected:", msg, flush=True)
    assert ei.value.status == status, msg
    assert text in msg, msg


@pytest.mark.parametrize("paged", [False, True])
def test_valid_batches_give_the_same_bits(paged, monkeypatch):
    print(f"case validate valid paged={paged}", flush=True)
    wl = small()
    outs = []
    for on in (False, True):
        if on:
            monkeypatch.setenv("DFLASH_VALIDATE", "1")
        dp = DevicePath(wl, paged=paged)
        dp.prepare_context()  # K-only norm + RoPE (positions), then the scatter when paged
        dp.step_fused()
        fused = dp.out.clone()
        dp.step()  # standalone norm + RoPE of q and k, then the attention
        torch.cuda.synchronize()
        outs.append((fused.view(torch.int16), dp.out.view(torch.int16)))
    assert torch.equal(outs[0][0], outs[1][0]), "fused"
    assert torch.equal(outs[0][1], outs[1][1]), "unfused"


def test_context_kv_valid_batch_gives_the_same_bits(monkeypatch):
    print("case validate context_kv valid", flush=True)
    wl = make_workload("ctx_kv", num_reqs=2, ctx_len=300, hidden=512)
    res = []
    for on in (False, True):
        if on:
            monkeypatch.setenv("DFLASH_VALIDATE", "1")
        dp = DevicePath(wl)
        dp.prepare_context()
        torch.cuda.synchronize()
        res.append((dp.k_ctx.view(torch.int16).clone(), dp.v_ctx.view(torch.int16).clone()))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])


def test_decreasing_context_lengths(validate):
    print("case validate cu_ctx decreasing", flush=True)
    wl = small()
    dp = DevicePath(wl, host_lengths=False)
    dp.prepare_context()
    c = dp.cu_ctx.clone()
    c[1] = c[2] + 1  # request 0 now ends after request 1 does
    dp.cu_ctx = c
    rejected(dp.attention_fused, B.DFLASH_ERR_INVALID_ARG, "cu_ctx_lens decreases at request 1")


def test_context_lengths_not_ending_at_total(validate):
    print("case validate cu_ctx end", flush=True)
    wl = small()
    dp = DevicePath(wl, host_lengths=False)
    dp.prepare_context()
    c = dp.cu_ctx.clone()
    c[-1] -= 1
    dp.cu_ctx = c
    rejected(dp.attention, B.DFLASH_ERR_INVALID_ARG, f"cu_ctx_lens ends at {wl.total_ctx - 1}")


def test_block_longer_than_max_blk_len(validate):
    print("case validate cu_blk long block", flush=True)
    wl = small()
    dp = DevicePath(wl, host_lengths=False)
    dp.prepare_context()
    c = dp.cu_blk.clone()
    c[1] += 4  # request 0: 20 block rows, more than max_blk_len 16
    dp.cu_blk = c
    rejected(dp.attention_fused, B.DFLASH_ERR_INVALID_ARG, "request 0 has 20 rows in cu_blk_lens")


def test_device_lengths_differ_from_host_copies(validate):
    print("case validate host/device lengths", flush=True)
    wl = small()
    dp = DevicePath(wl)  # host copies go with the parameters
    dp.prepare_context()
    c = dp.cu_ctx.clone()
    c[1] += 1  # still a valid batch by itself, but not the one the host planned
    dp.cu_ctx = c
    rejected(dp.attention_fused, B.DFLASH_ERR_INVALID_ARG,
             "device cu_ctx_lens[1] = %d differs from the host copy" % int(wl.cu_ctx[1] + 1))


@pytest.mark.parametrize("bad", ["past_end", "negative"])
def test_prologue_positions_out_of_range(validate, bad):
    print(f"case validate prologue positions {bad}", flush=True)
    wl = small()
    dp = DevicePath(wl)
    dp.prepare_context()
    value = dp.max_pos if bad == "past_end" else -3
    dp.blk_pos[5] = value  # the prologue holds this tensor's address
    rejected(dp.attention_fused, B.DFLASH_ERR_INVALID_ARG, f"positions[5] = {value} is outside")


def test_standalone_norm_rope_positions_out_of_range(validate):
    print("case validate qk_norm_rope positions", flush=True)
    wl = small()
    dp = DevicePath(wl)
    dp.ctx_pos[7] = dp.max_pos + 10
    rejected(dp.prepare_context, B.DFLASH_ERR_INVALID_ARG, "qk_norm_rope: positions[7]")


def test_context_kv_positions_out_of_range(validate):
    print("case validate context_kv positions", flush=True)
    wl = make_workload("ctx_kv", num_reqs=2, ctx_len=300, hidden=512)
    dp = DevicePath(wl)
    dp.ctx_pos[11] = -1
    rejected(dp.prepare_context, B.DFLASH_ERR_INVALID_ARG, "context_kv: positions[11] = -1")


def test_page_id_out_of_range(validate):
    print("case validate page id", flush=True)
    wl = small()
    dp = DevicePath(wl, paged=True)
    dp.prepare_context()
    dp.block_table[2, 1] = dp.num_pages
    rejected(dp.attention_fused, B.DFLASH_ERR_INVALID_ARG,
             f"block_table[2][1] = {dp.num_pages} is outside [0, {dp.num_pages})")


def test_scatter_slots(validate):
    print("case validate scatter slots", flush=True)
    wl = small()
    dp = DevicePath(wl, paged=True)
    s = dp.slot_mapping
    s[2] = -1  # a padding row: allowed, written nowhere
    dp.prepare_context()
    s[9] = s[4]
    rejected(dp.prepare_context, B.DFLASH_ERR_INVALID_ARG, "is written by more than one row")


def test_captured_stream_is_refused(validate):
    print("case validate under capture", flush=True)
    wl = small()
    dp = DevicePath(wl)
    dp.prepare_context()
    scratch = torch.zeros(16, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    err = None
    with torch.cuda.graph(g):
        scratch.add_(1.0)  # the graph holds one plain node
        try:
            dp.attention_fused()
        except B.DflashError as e:
            err = e
    torch.cuda.synchronize()
    assert err is not None and err.status == B.DFLASH_ERR_UNSUPPORTED, err
    assert "captured" in str(err)
