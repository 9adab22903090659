"""A whole propose step (preparation, fc combine, context K/V appended to the
paged store, block q/k/v, paged attention planned on the device, o_proj)
captured once into a HIP graph and replayed over several steps with its
inputs refreshed in place: every replay matches the same step run eagerly on
a twin with the same weights, bitwise (outputs, prepared metadata and the
paged store), with unrelated device work between the replays; and every
replay's attention output and o_proj output match the fp64 oracle (fc
combine of the verified rows, context K/V of every kept row so far, the draft
layer's attention block over them) within the bf16 output bars."""
import numpy as np
import pytest
import torch

from block_diffusion_draft_dflash_amd import binding as B
from block_diffusion_draft_dflash_amd.pipeline import DraftStep, to_host_f64

pytestmark = pytest.mark.gpu

R, NQPR, ROWS = 4, 8, 8


def _inputs(rng, ds, ctx_len, first):
    pos = np.concatenate([np.arange(c, c + ROWS) for c in ctx_len])
    rejected = np.zeros(R, np.int64) if first else rng.integers(0, ROWS, size=R)
    sampled = np.zeros(R, np.int64) if first else np.ones(R, np.int64)   # a prefill step samples nothing
    last = rng.integers(0, 1000, size=R)
    aux = rng.standard_normal((R * ROWS, ds.h * ds.taps), dtype=np.float32)
    return (pos, rejected, sampled, last, aux), rejected


class _OracleStep:
    """The oracle's view of the step: every request's context grows by the
    combined features of its kept verified rows (positions 0, 1, ... in
    order), and the block (positions right after the kept context) goes
    through the draft layer's attention block."""

    def __init__(self, ds):
        f = to_host_f64
        self.ds = ds
        self.w = dict(fc=f(ds.w_fc), hnw=f(ds.hnw), knw=f(ds.knw), qnw=f(ds.qnw), inw=f(ds.in_norm_w),
                      wk=f(ds.w_k), wv=f(ds.w_v), wqkv=f(ds.w_qkv), wo=f(ds.w_o), blk=f(ds.blk_hidden))
        self.feats = [np.zeros((0, ds.h)) for _ in range(ds.r)]

    def step(self, aux, rejected):
        from oracle import dflash_oracle as O
        ds, w = self.ds, self.w
        comb = O.fc_combine(O.bf16_round(aux), w["fc"])
        for i in range(ds.r):
            keep = ds.rows - int(rejected[i])
            self.feats[i] = np.concatenate([self.feats[i], comb[i * ds.rows:i * ds.rows + keep]])
        ctx = np.array([len(x) for x in self.feats])
        cpos = np.concatenate([np.arange(c) for c in ctx])
        k_hat, v_ctx = O.context_kv(np.concatenate(self.feats), w["hnw"], w["wk"], w["wv"], w["knw"],
                                    cpos, ds.hkv, ds.dh, ds.eps, 1e6)
        qpos = np.concatenate([np.arange(c, c + ds.nqpr) for c in ctx])
        cu_c = np.concatenate([[0], np.cumsum(ctx)])
        cu_b = np.arange(ds.r + 1) * ds.nqpr
        o, _, _, _, _, attn = O.draft_layer_attention(
            w["blk"], None, w["inw"], w["wqkv"], w["wo"], qpos, k_hat, v_ctx, cu_c, cu_b, w["qnw"],
            w["knw"], ds.hq, ds.hkv, ds.dh, ds.eps, 1e6, ds.dh ** -0.5)
        return attn, o


def _assert_bars(got, ref, tag):
    err = np.abs(to_host_f64(got).reshape(ref.shape) - ref)
    print(f"[{tag}] max abs {err.max():.3e} mean abs {err.mean():.3e}", flush=True)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3, tag


def _same(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


def test_draft_step_graph_replay():
    print("case draft step graph replay", flush=True)
    eager = DraftStep(R, NQPR, ROWS, seed=3)
    graph = DraftStep(R, NQPR, ROWS, seed=3)
    ref = _OracleStep(graph)
    rng = np.random.default_rng(9)
    ctx = np.zeros(R, np.int64)
    # cold -> warm: the first (prefill) step eagerly on both
    inp, rej = _inputs(rng, eager, ctx, True)
    eager.set_step(*inp)
    graph.set_step(*inp)
    eager.run()
    graph.run()
    torch.cuda.synchronize()
    attn_ref, o_ref = ref.step(inp[4], rej)
    _assert_bars(graph.attn, attn_ref, "draft step 0 (eager) attention vs oracle")
    _assert_bars(graph.o, o_ref, "draft step 0 (eager) o_proj vs oracle")
    ctx += ROWS - rej
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graph.run()
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device="cuda")
    for step in range(1, 5):
        inp, rej = _inputs(rng, eager, ctx, False)
        eager.set_step(*inp)
        graph.set_step(*inp)
        scratch.mul_(1.0001).add_(0.5)          # unrelated eager work between replays
        eager.run()
        g.replay()
        torch.cuda.synchronize()
        for n in B.PREP_OUT:
            assert _same(eager.outs[n], graph.outs[n]), f"step {step}: {n} differs"
        assert torch.equal(eager.outs["ctx_cu"][1:].cpu() - eager.outs["ctx_cu"][:-1].cpu(),
                           torch.from_numpy((ctx + ROWS - rej).astype(np.int32))), "kept context lengths"
        for name in ("k_pool", "v_pool", "q", "attn", "o"):
            assert _same(getattr(eager, name), getattr(graph, name)), f"step {step}: {name} differs"
        assert not torch.isnan(graph.o.float()).any()
        attn_ref, o_ref = ref.step(inp[4], rej)
        _assert_bars(graph.attn, attn_ref, f"draft step {step} (replay) attention vs oracle")
        _assert_bars(graph.o, o_ref, f"draft step {step} (replay) o_proj vs oracle")
        ctx += ROWS - rej
        print(f"[draft step {step}] context rows {ctx.tolist()}: replay == eager", flush=True)
