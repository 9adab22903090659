"""The propose step's data flow on the GPU: dflash_prepare_inputs (bit-exact
against the oracle), dflash_fc_combine (per-element bound), and two steps of
the whole flow -- fc combine of the target's tapped features, context K/V of
the kept rows appended to a paged store at the prepared slots, the anchor +
mask block attending over the context -- against the oracle.

fc_combine bound: the aux rounding to bf16 is part of the definition (both
sides round to nearest even); the GPU accumulates in f32 (<= 2^-11 sum |a w|
over K <= 2^14 terms with split partial sums) and rounds the output once:
|g - o| <= 2^-11 sum_k |a_k w_nk| + 2^-8 |o| + 1e-6.
"""
import os

import numpy as np
import pytest
import torch

from block_diffusion_draft_dflash_amd import binding as B
from block_diffusion_draft_dflash_amd.pipeline import bits_to_device, to_host_f64
from block_diffusion_draft_dflash_amd.workloads import bf16_bits_to_f32, f32_to_bf16_bits

pytestmark = pytest.mark.gpu



def _run_prep(batch, sentinel=-777):
    """Run dflash_prepare_inputs on ``batch`` (the oracle's keyword arguments);
    outputs start filled with a sentinel so unwritten entries show."""
    dev = "cuda"
    r = len(batch["idx_mapping"])
    nqpr, nspec = batch["num_query_per_req"], batch["num_speculative_steps"]
    ntgt = int(batch["target_query_start_loc"][-1])
    bt = np.asarray(batch["block_table"], dtype=np.int64).reshape(r, -1)
    t = lambda a, name: torch.tensor(np.asarray(a, dtype=np.int32), device=dev)
    ins = {n: t(batch[n] if n != "block_table" else bt, n) for n in B.PREP_IN}
    sizes = dict(input_ids=r * nqpr, query_positions=r * nqpr,
                 query_start_loc=batch["max_num_reqs"] + 1, seq_lens=batch["max_num_reqs"],
                 query_slot_mapping=batch["max_num_tokens"], context_positions=ntgt,
                 context_slot_mapping=ntgt, sample_indices=batch["max_num_reqs"] * nspec,
                 sample_pos=batch["max_num_reqs"] * nspec,
                 sample_idx_mapping=batch["max_num_reqs"] * nspec,
                 ctx_cu=batch["max_num_reqs"] + 1)
    outs = {n: torch.full((sizes[n],), sentinel, dtype=torch.int32, device=dev) for n in B.PREP_OUT}
    p = B.PrepareParams(r, batch["max_num_reqs"], batch["max_num_tokens"], nqpr, nspec,
                        batch["block_size"], bt.shape[1], batch["max_model_len"],
                        batch["mask_token_id"], int(batch["sample_from_anchor"]),
                        len(batch["last_sampled"]), ntgt)
    B.dflash_prepare_inputs(p, ins, outs)
    torch.cuda.synchronize()
    return {n: v.cpu().numpy().astype(np.int64) for n, v in outs.items()}


def _hand_batch(sample_from_anchor=False, max_model_len=100):
    nqpr = 3
    return dict(idx_mapping=[1, 0], target_query_start_loc=[0, 3, 4], target_positions=[5, 6, 7, 0],
                num_rejected=[1, 0], num_sampled=[1, 0], last_sampled=[11, 42],
                next_prefill_tokens=[17, 99], block_table=[[9, 3, 7], [2, 5, 6]],
                num_query_per_req=nqpr, num_speculative_steps=nqpr - (0 if sample_from_anchor else 1),
                block_size=4, max_num_reqs=3, max_num_tokens=8, max_model_len=max_model_len,
                mask_token_id=-5, sample_from_anchor=sample_from_anchor)


def _random_batch(seed, sample_from_anchor, num_reqs=None):
    rng = np.random.default_rng(seed)
    r = int(rng.integers(1, 41)) if num_reqs is None else num_reqs
    nqpr = int(rng.integers(1, 17))
    if not sample_from_anchor:
        nqpr = max(nqpr, 2)
    bs = int(rng.choice([1, 4, 16]))
    states = int(r + rng.integers(0, 5))
    t_req = rng.integers(1, 40, size=r)
    t_req[rng.random(r) < 0.2] = int(rng.integers(100, 400))      # a few prefill chunks
    start_pos = rng.integers(0, 3000, size=r)
    pos = np.concatenate([np.arange(s, s + n) for s, n in zip(start_pos, t_req)])
    rej = np.array([int(rng.integers(0, n)) for n in t_req])          # keeps at least one row
    stride = int(rng.integers(1, 3200 // bs + 2))                     # some positions past the table
    bt = rng.integers(0, 100000, size=(r, stride))
    return dict(idx_mapping=rng.permutation(states)[:r].tolist(),
                target_query_start_loc=np.concatenate([[0], np.cumsum(t_req)]).tolist(),
                target_positions=pos.tolist(), num_rejected=rej.tolist(),
                num_sampled=rng.integers(0, 3, size=r).tolist(),
                last_sampled=rng.integers(0, 150000, size=states).tolist(),
                next_prefill_tokens=rng.integers(0, 150000, size=states).tolist(),
                block_table=bt, num_query_per_req=nqpr,
                num_speculative_steps=nqpr - (0 if sample_from_anchor else 1), block_size=bs,
                max_num_reqs=r + int(rng.integers(0, 9)),
                max_num_tokens=r * nqpr + int(rng.integers(0, 33)),
                max_model_len=int(rng.integers(1000, 4000)), mask_token_id=151665,
                sample_from_anchor=sample_from_anchor)


def _assert_prep_equal(got, want, tag):
    for n in B.PREP_OUT:
        assert np.array_equal(got[n], want[n]), f"{tag}: {n} differs"


@pytest.mark.parametrize("anchor", [False, True])
def test_prepare_inputs_hand_example(anchor):
    from oracle import dflash_oracle as O
    print(f"case prepare hand anchor={anchor}", flush=True)
    b = _hand_batch(sample_from_anchor=anchor, max_model_len=9 if anchor else 100)
    _assert_prep_equal(_run_prep(b), O.prepare_dflash_inputs(**b), "hand")


# 12 batches by default; DFLASH_RANDOM_CASES=N runs the first N seeds
@pytest.mark.parametrize("seed", range(int(os.environ.get("DFLASH_RANDOM_CASES", "12"))))
def test_prepare_inputs_random(seed):
    from oracle import dflash_oracle as O
    anchor = bool(seed % 2)
    print(f"case prepare random seed={seed} anchor={anchor}", flush=True)
    b = _random_batch(100 + seed, anchor)
    _assert_prep_equal(_run_prep(b), O.prepare_dflash_inputs(**b), f"seed {seed}")


@pytest.mark.parametrize("num_reqs", [256, 600])
def test_prepare_inputs_many_requests(num_reqs):
    # the cumulative context lengths are scanned 256 requests at a time: a
    # full chunk, then several chunks with a ragged tail
    from oracle import dflash_oracle as O
    print(f"case prepare many requests R={num_reqs}", flush=True)
    b = _random_batch(500 + num_reqs, num_reqs % 2 == 0, num_reqs=num_reqs)
    _assert_prep_equal(_run_prep(b), O.prepare_dflash_inputs(**b), f"R={num_reqs}")


@pytest.mark.parametrize("shape", [(7, 256, 3), (128, 512, 5), (300, 128, 2), (64, 2048, 6)])
def test_fc_combine_vs_oracle(shape):
    from oracle import dflash_oracle as O
    t, h, taps = shape
    print(f"case fc_combine {shape}", flush=True)
    rng = np.random.default_rng(sum(shape))
    aux = rng.standard_normal((t, h * taps), dtype=np.float32) * np.float32(2.0)
    w_bits = f32_to_bf16_bits(rng.standard_normal((h, h * taps), dtype=np.float32) * np.float32(0.02))
    out = torch.full((t, h), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = B.alloc_workspace(B.dflash_fc_combine_workspace_size(t, h, taps))
    B.dflash_fc_combine(torch.from_numpy(aux).cuda(), bits_to_device(w_bits), out, ws)
    torch.cuda.synchronize()
    a = O.bf16_round(aux)
    w = bf16_bits_to_f32(w_bits).astype(np.float64)
    ref = O.fc_combine(a, w)
    bound = 2.0 ** -11 * (np.abs(a) @ np.abs(w).T) + 2.0 ** -8 * np.abs(ref) + 1e-6
    err = np.abs(to_host_f64(out) - ref)
    print(f"[fc {shape}] max abs {err.max():.3e} worst err/bound {(err / bound).max():.3f}", flush=True)
    assert (err <= bound).all()


# ---------------------------------------------------------------- two steps of the data flow

H, TAPS, HQ, HKV, DH, PAGE = 256, 3, 4, 2, 128, 16
EPS, THETA = 1e-6, 1e6


class _Flow:
    """Per-request context over a paged store, grown by propose steps."""

    def __init__(self, nreq, seed):
        self.rng = np.random.default_rng(seed)
        self.r = nreq
        self.stride = 24                                      # pages per request (384 rows)
        self.pages = nreq * self.stride + 7
        perm = self.rng.permutation(self.pages)[:nreq * self.stride]
        self.bt = perm.reshape(nreq, self.stride).astype(np.int64)
        bits = lambda shape, s: f32_to_bf16_bits(self.rng.standard_normal(shape, dtype=np.float32)
                                                 * np.float32(s))
        self.w_fc = bits((H, H * TAPS), 0.05)
        self.w_k = bits((HKV * DH, H), 0.05)
        self.w_v = bits((HKV * DH, H), 0.05)
        f = lambda a, lo, hi: bf16_bits_to_f32(f32_to_bf16_bits(
            self.rng.uniform(lo, hi, a).astype(np.float32)))
        self.hnw, self.knw, self.qnw = f(H, 0.5, 1.5), f(DH, 0.5, 1.5), f(DH, 0.5, 1.5)
        dev = "cuda"
        self.k_pool = torch.full((self.pages, PAGE, HKV, DH), float("nan"), dtype=torch.bfloat16, device=dev)
        self.v_pool = torch.full_like(self.k_pool, float("nan"))
        self.ctx_len = np.zeros(nreq, np.int64)                # kept context rows per request
        self.ctx_feats = [np.zeros((0, H)) for _ in range(nreq)]  # oracle: combined rows kept
        self.last_sampled = self.rng.integers(0, 1000, size=nreq)

    def step(self, t_req, rejected, nqpr):
        """One propose step: the target verified t_req[r] rows of request r at
        positions ctx_len[r].., of which the last rejected[r] are rolled back."""
        from oracle import dflash_oracle as O
        dev = "cuda"
        r = self.r
        pos = np.concatenate([np.arange(c, c + n) for c, n in zip(self.ctx_len, t_req)])
        ntgt = int(np.sum(t_req))
        aux = self.rng.standard_normal((ntgt, H * TAPS), dtype=np.float32)
        batch = dict(idx_mapping=list(range(r)),
                     target_query_start_loc=np.concatenate([[0], np.cumsum(t_req)]).tolist(),
                     target_positions=pos.tolist(), num_rejected=list(rejected),
                     num_sampled=[1] * r, last_sampled=self.last_sampled.tolist(),
                     next_prefill_tokens=[0] * r, block_table=self.bt, num_query_per_req=nqpr,
                     num_speculative_steps=nqpr - 1, block_size=PAGE, max_num_reqs=r,
                     max_num_tokens=r * nqpr, max_model_len=1 << 20, mask_token_id=7,
                     sample_from_anchor=False)
        prep = _run_prep(batch)
        ref_prep = O.prepare_dflash_inputs(**batch)
        _assert_prep_equal(prep, ref_prep, "flow prep")
        # fc combine of the tapped features, then context K/V of every verified
        # row written to its slot (rejected rows too: they are never read)
        comb = torch.empty((ntgt, H), dtype=torch.bfloat16, device=dev)
        B.dflash_fc_combine(torch.from_numpy(aux).to(dev), bits_to_device(self.w_fc), comb,
                            B.alloc_workspace(B.dflash_fc_combine_workspace_size(ntgt, H, TAPS)))
        k_new = torch.empty((ntgt, HKV, DH), dtype=torch.bfloat16, device=dev)
        v_new = torch.empty_like(k_new)
        table = torch.empty((1 << 12, DH // 2, 2), dtype=torch.float32, device=dev)
        B.dflash_rope_table(table, 1 << 12, DH, THETA)
        ctx_pos = torch.from_numpy(prep["context_positions"].astype(np.int32)).to(dev)
        B.dflash_context_kv(comb, torch.from_numpy(self.hnw).to(dev), bits_to_device(self.w_k),
                            bits_to_device(self.w_v), torch.from_numpy(self.knw).to(dev), ctx_pos,
                            HKV, DH, EPS, table, k_new, v_new,
                            B.alloc_workspace(B.dflash_context_kv_workspace_size(ntgt, H, HKV, DH)))
        slots = torch.from_numpy(prep["context_slot_mapping"].astype(np.int32)).to(dev)
        B.dflash_kv_scatter(k_new, v_new, slots, self.k_pool, self.v_pool)
        # oracle: the combined features of the kept rows extend each request's context
        comb_ref = O.fc_combine(O.bf16_round(aux), bf16_bits_to_f32(self.w_fc).astype(np.float64))
        cu = batch["target_query_start_loc"]
        for i in range(r):
            keep = t_req[i] - rejected[i]
            self.ctx_feats[i] = np.concatenate([self.ctx_feats[i], comb_ref[cu[i]:cu[i] + keep]])
            self.ctx_len[i] += keep
        return prep

    def attend(self, prep, nqpr):
        """The anchor + mask block of every request over its kept context."""
        from oracle import dflash_oracle as O
        dev = "cuda"
        r = self.r
        ctx_lens = prep["seq_lens"][:r] - nqpr
        assert np.array_equal(ctx_lens, self.ctx_len), "seq_lens disagree with the kept context"
        t = r * nqpr
        q = f32_to_bf16_bits(self.rng.standard_normal((t, HQ, DH), dtype=np.float32))
        kb = f32_to_bf16_bits(self.rng.standard_normal((t, HKV, DH), dtype=np.float32))
        vb = f32_to_bf16_bits(self.rng.standard_normal((t, HKV, DH), dtype=np.float32))
        cu_ctx = np.concatenate([[0], np.cumsum(ctx_lens)]).astype(np.int32)
        cu_blk = (np.arange(r + 1) * nqpr).astype(np.int32)
        qpos = prep["query_positions"].astype(np.int32)
        table = torch.empty((1 << 12, DH // 2, 2), dtype=torch.float32, device=dev)
        B.dflash_rope_table(table, 1 << 12, DH, THETA)
        p = B.make_block_attn_params(r, HQ, HKV, DH, B.DFLASH_BF16, int(cu_ctx[-1]), t, nqpr,
                                     DH ** -0.5, host_cu_ctx_lens=cu_ctx, host_cu_blk_lens=cu_blk)
        # the prologue and paged-store records hold raw device pointers: keep
        # the tensors they point to alive until the call has run
        qnw_d, knw_d = torch.from_numpy(self.qnw).to(dev), torch.from_numpy(self.knw).to(dev)
        qpos_d = torch.from_numpy(qpos).to(dev)
        bt_d = torch.from_numpy(self.bt.astype(np.int32)).to(dev)
        pro = B.make_qk_prologue(qnw_d, knw_d, qpos_d, table, EPS)
        pg = B.make_paged_ctx(bt_d, self.pages)
        out = torch.empty((t, HQ, DH), dtype=torch.bfloat16, device=dev)
        B.dflash_block_attention_paged(p, pg, torch.from_numpy(cu_ctx).to(dev),
                                       torch.from_numpy(cu_blk).to(dev), bits_to_device(q),
                                       bits_to_device(kb), bits_to_device(vb), self.k_pool,
                                       self.v_pool, out,
                                       B.alloc_workspace(B.dflash_block_attention_paged_workspace_size(p)),
                                       prologue=pro)
        torch.cuda.synchronize()
        feats = np.concatenate(self.ctx_feats)
        cpos = np.concatenate([np.arange(c) for c in ctx_lens])
        k_hat, v_ctx = O.context_kv(feats, self.hnw, bf16_bits_to_f32(self.w_k), bf16_bits_to_f32(self.w_v),
                                    self.knw, cpos, HKV, DH, EPS, THETA)
        ref, _, _ = O.draft_block_attention(bf16_bits_to_f32(q), bf16_bits_to_f32(kb), bf16_bits_to_f32(vb),
                                            qpos, k_hat, v_ctx, cu_ctx, cu_blk, self.qnw, self.knw,
                                            EPS, THETA, DH ** -0.5)
        err = np.abs(to_host_f64(out) - ref)
        print(f"[flow attention] max abs {err.max():.3e} mean abs {err.mean():.3e}", flush=True)
        assert not torch.isnan(out.float()).any()
        assert err.max() <= 2e-2 and err.mean() <= 2e-3


def test_propose_flow_two_steps():
    print("case propose flow", flush=True)
    fl = _Flow(nreq=4, seed=21)
    nqpr = 8
    # step 0: prefill chunks (nothing rejected); step 1: verification of the
    # previous block (1 + k rows) with some drafts rejected
    prep0 = fl.step(t_req=[37, 1, 120, 16], rejected=[0, 0, 0, 0], nqpr=nqpr)
    fl.attend(prep0, nqpr)
    prep1 = fl.step(t_req=[nqpr] * 4, rejected=[3, 0, 7, 5], nqpr=nqpr)
    fl.attend(prep1, nqpr)


# (the last case: 128-wide tiles, K's and V's weights as the two halves of N)
# (hidden 256 plans one K slice: the GEMM writes K and V itself and the
# q/k-norm kernel follows; the others sum split partials in the kernel that
# also applies the k-norm and RoPE)
@pytest.mark.parametrize("rows,hkv,h", [(1, 2, 512), (37, 2, 512), (255, 2, 512), (37, 4, 512),
                                        (37, 16, 8192), (37, 2, 256)])
def test_context_kv_few_rows_vs_oracle(rows, hkv, h):
    # calls of fewer than 256 rows (a step's appended rows) take the
    # projection-GEMM path (K and V in one product over the two weights);
    # scale-relative bound as for the large-row form
    _context_kv_vs_oracle(rows, hkv, h)


# the large-row form (256 rows and more: the fused MFMA GEMM) at hidden sizes
# of one, two and three 64-wide k-slices and up, whole and partial 256-row
# tiles, and K / V head counts of 2 to 8 (two heads per 256-column tile)
@pytest.mark.parametrize("rows,hkv,h", [(256, 2, 64), (300, 2, 128), (520, 4, 192), (777, 8, 1024),
                                        (1030, 2, 64)])
def test_context_kv_large_rows_shapes_vs_oracle(rows, hkv, h):
    _context_kv_vs_oracle(rows, hkv, h)


def _context_kv_vs_oracle(rows, hkv, h):
    from oracle import dflash_oracle as O
    print(f"case context_kv rows={rows} hkv={hkv} h={h}", flush=True)
    rng = np.random.default_rng(rows)
    dh = 128
    hid = f32_to_bf16_bits(rng.standard_normal((rows, h), dtype=np.float32))
    bits = lambda shape: f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(0.02))
    wk, wv = bits((hkv * dh, h)), bits((hkv * dh, h))
    f = lambda n: bf16_bits_to_f32(f32_to_bf16_bits(rng.uniform(0.5, 1.5, n).astype(np.float32)))
    hnw, knw = f(h), f(dh)
    pos = rng.integers(0, 5000, size=rows).astype(np.int32)
    dev = "cuda"
    table = torch.empty((8192, dh // 2, 2), dtype=torch.float32, device=dev)
    B.dflash_rope_table(table, 8192, dh, 1e6)
    k = torch.empty((rows, hkv, dh), dtype=torch.bfloat16, device=dev)
    v = torch.empty_like(k)
    args = lambda lo, hi, ko, vo: (bits_to_device(hid[lo:hi]), torch.from_numpy(hnw).to(dev),
                                   bits_to_device(wk), bits_to_device(wv), torch.from_numpy(knw).to(dev),
                                   torch.from_numpy(pos[lo:hi]).to(dev), hkv, dh, 1e-6, table, ko, vo,
                                   B.alloc_workspace(B.dflash_context_kv_workspace_size(hi - lo, h, hkv, dh)))
    B.dflash_context_kv(*args(0, rows, k, v))
    torch.cuda.synchronize()
    kr, vr = O.context_kv(bf16_bits_to_f32(hid), hnw, bf16_bits_to_f32(wk), bf16_bits_to_f32(wv), knw,
                          pos, hkv, dh, 1e-6, 1e6)
    for name, g, o in (("K", k, kr), ("V", v, vr)):
        rel = np.abs(to_host_f64(g) - o).max() / np.abs(o).max()
        print(f"[context_kv rows={rows} {name}] scale-relative max err {rel:.3e}", flush=True)
        assert rel <= 1e-2
    if rows > 1:
        # row independence within this form: calls over row chunks of the same
        # form (fewer than 256 rows, else 256-row windows at both ends; the
        # two forms add in different orders)
        cut = rows // 3
        chunks = ((0, cut), (cut, rows)) if rows < 256 else ((0, 256), (rows - 256, rows))
        for lo, hi in chunks:
            kc = torch.empty((hi - lo, hkv, dh), dtype=torch.bfloat16, device=dev)
            vc = torch.empty_like(kc)
            B.dflash_context_kv(*args(lo, hi, kc, vc))
            torch.cuda.synchronize()
            assert torch.equal(kc.view(torch.int16), k[lo:hi].view(torch.int16))
            assert torch.equal(vc.view(torch.int16), v[lo:hi].view(torch.int16))
