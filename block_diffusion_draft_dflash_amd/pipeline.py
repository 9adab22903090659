"""Device-side driver of one synthetic batch through libdflash.

Uploads a :class:`~block_diffusion_draft_dflash_amd.workloads.Workload` to the
GPU, builds the RoPE cos/sin cache and the workspaces, and runs the path
through the C ABI:

* context rows: ``dflash_context_kv`` from hidden states when the workload has
  them, else the K-only ``dflash_qk_norm_rope`` on the raw context keys;
* the step: ``dflash_qk_norm_rope`` on the block's q and k (in place), then
  ``dflash_block_attention`` over [context; block]; or the one fused call;
* the draft layer around it (:class:`LayerPath`): ``dflash_block_qkv`` (input
  norm and merged q/k/v projection of the block rows), the fused attention,
  ``dflash_o_proj``;
* a whole propose step (:class:`DraftStep`), capturable into a HIP graph.

By default the host copies of the cumulative lengths go with the attention
parameters (the work split is then planned on the host); ``host_lengths=False``
leaves the planning to the kernels.

Only argument marshalling happens here; every step runs in the HIP library.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import binding as B
from .workloads import LayerInputs, Workload, bf16_bits_to_f32, f32_to_bf16_bits


def to_device(x: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Upload float32 values (bf16-representable for bf16) without rounding changes."""
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x)
        return torch.from_numpy(bits.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def bits_to_device(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def to_host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


class DevicePath:
    def __init__(self, wl: Workload, device: str = "cuda", split_keys: int = 0,
                 max_pos: Optional[int] = None, host_lengths: bool = True, paged: bool = False,
                 spare_pages: int = 5):
        self.wl = wl
        self.device = device
        dt = wl.dtype
        self.dtype_code = B.DFLASH_BF16 if dt == "bf16" else B.DFLASH_F32
        i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)
        self.cu_ctx = i32(wl.cu_ctx)
        self.cu_blk = i32(wl.cu_blk)
        self.ctx_pos = i32(wl.ctx_positions)
        self.blk_pos = i32(wl.blk_positions)
        self.q = to_device(wl.q, dt, device)
        self.k_blk = to_device(wl.k_blk, dt, device)
        self.v_blk = to_device(wl.v_blk, dt, device)
        f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
        self.q_norm_w = f32(wl.q_norm_w)
        self.k_norm_w = f32(wl.k_norm_w)
        if max_pos is None:
            mp = 1
            if wl.ctx_positions.size:
                mp = max(mp, int(wl.ctx_positions.max()) + 1)
            if wl.blk_positions.size:
                mp = max(mp, int(wl.blk_positions.max()) + 1)
            max_pos = mp
        self.max_pos = max_pos
        self.rope = torch.empty((max_pos, wl.dh // 2, 2), dtype=torch.float32, device=device)
        B.dflash_rope_table(self.rope, max_pos, wl.dh, wl.theta)
        tc = wl.total_ctx
        if wl.hidden is not None:
            self.hidden = bits_to_device(wl.hidden, device)
            self.hidden_norm_w = f32(wl.hidden_norm_w)
            self.w_k = bits_to_device(wl.w_k, device)
            self.w_v = bits_to_device(wl.w_v, device)
            tdt = torch.bfloat16
            self.k_ctx = torch.empty((tc, wl.hkv, wl.dh), dtype=tdt, device=device)
            self.v_ctx = torch.empty((tc, wl.hkv, wl.dh), dtype=tdt, device=device)
            ckv_ws = B.dflash_context_kv_workspace_size(tc, wl.hidden_size, wl.hkv, wl.dh)
            self.ckv_ws = B.alloc_workspace(ckv_ws, device)
            self.k_ctx_raw = None
        else:
            self.hidden = None
            self.k_ctx_raw = to_device(wl.k_ctx, dt, device)
            self.k_ctx = self.k_ctx_raw.clone()
            self.v_ctx = to_device(wl.v_ctx, dt, device)
        self.out = torch.zeros_like(self.q)
        # raw copies for the fused path (never modified)
        self.q_raw = self.q.clone()
        self.k_blk_raw = self.k_blk.clone()
        self.prologue = B.make_qk_prologue(self.q_norm_w, self.k_norm_w, self.blk_pos, self.rope,
                                           wl.eps)
        self.params = B.make_block_attn_params(
            wl.num_reqs, wl.hq, wl.hkv, wl.dh, self.dtype_code, tc, wl.total_blk,
            int(wl.blk_lens.max()) if wl.num_reqs else 0, wl.scale, wl.causal, wl.window,
            split_keys,
            host_cu_ctx_lens=wl.cu_ctx if host_lengths else None,
            host_cu_blk_lens=wl.cu_blk if host_lengths else None)
        self.paged = paged
        if paged:
            self._init_paged(spare_pages)
            self.ws = B.alloc_workspace(
                B.dflash_block_attention_paged_workspace_size(self.params), device)
        else:
            self.ws = B.alloc_workspace(B.dflash_block_attention_workspace_size(self.params), device)

    def _init_paged(self, spare_pages: int) -> None:
        """A paged store holding the context rows: pages handed out in a seeded
        random order (so a request's pages are scattered over the pool), spare
        pages left unused, and every slot filled with NaN first, so a read of a
        slot the table does not map shows up in the output."""
        wl = self.wl
        page = 16
        npages_r = [(int(c) + page - 1) // page for c in wl.ctx_lens]
        total = sum(npages_r) + spare_pages
        perm = np.random.default_rng(4242).permutation(total).astype(np.int32)
        maxp = max(1, max(npages_r) if npages_r else 1)
        bt = np.full((wl.num_reqs, maxp), -1, dtype=np.int32)
        slots = np.empty(wl.total_ctx, dtype=np.int32)
        nxt = 0
        for r in range(wl.num_reqs):
            c0 = int(wl.cu_ctx[r])
            for pidx in range(npages_r[r]):
                bt[r, pidx] = perm[nxt]
                nxt += 1
            for j in range(int(wl.ctx_lens[r])):
                slots[c0 + j] = bt[r, j // page] * page + j % page
        self.num_pages = total
        self.block_table = torch.from_numpy(bt).to(self.device)
        self.slot_mapping = torch.from_numpy(slots).to(self.device)
        dt = self.k_ctx.dtype
        shape = (total, page, wl.hkv, wl.dh)
        self.k_pool = torch.full(shape, float("nan"), dtype=dt, device=self.device)
        self.v_pool = torch.full(shape, float("nan"), dtype=dt, device=self.device)
        self.pg = B.make_paged_ctx(self.block_table, total, page)

    # ---------------------------------------------------------------- context
    def prepare_context(self) -> None:
        """Produce the normed + rotated context keys (and V for hidden-state input);
        with a paged store, then scatter them to their pool slots."""
        self._prepare_packed_context()
        if self.paged and self.wl.total_ctx:
            B.dflash_kv_scatter(self.k_ctx, self.v_ctx, self.slot_mapping, self.k_pool, self.v_pool)

    def _prepare_packed_context(self) -> None:
        wl = self.wl
        if self.hidden is not None:
            B.dflash_context_kv(self.hidden, self.hidden_norm_w, self.w_k, self.w_v,
                                self.k_norm_w, self.ctx_pos, wl.hkv, wl.dh, wl.eps, self.rope,
                                self.k_ctx, self.v_ctx, self.ckv_ws)
        else:
            self.k_ctx.copy_(self.k_ctx_raw)
            if wl.total_ctx:
                B.dflash_qk_norm_rope(None, self.k_ctx, None, self.k_norm_w, self.ctx_pos,
                                      wl.eps, self.rope)

    # ---------------------------------------------------------------- step
    def qk_norm_rope(self) -> None:
        if self.wl.total_blk:
            B.dflash_qk_norm_rope(self.q, self.k_blk, self.q_norm_w, self.k_norm_w,
                                  self.blk_pos, self.wl.eps, self.rope)

    def _attn(self, q, k_blk, prologue) -> None:
        has_ctx = self.wl.total_ctx > 0
        if self.paged:
            B.dflash_block_attention_paged(self.params, self.pg, self.cu_ctx, self.cu_blk, q, k_blk,
                                           self.v_blk, self.k_pool if has_ctx else None,
                                           self.v_pool if has_ctx else None, self.out, self.ws,
                                           prologue=prologue)
        else:
            B.dflash_block_attention(self.params, self.cu_ctx, self.cu_blk, q, k_blk, self.v_blk,
                                     self.k_ctx if has_ctx else None,
                                     self.v_ctx if has_ctx else None, self.out, self.ws,
                                     prologue=prologue)

    def attention(self) -> None:
        self._attn(self.q, self.k_blk, None)

    def attention_fused(self) -> None:
        """Block attention with the q/k norm + RoPE fused in (raw q and k_blk)."""
        self._attn(self.q_raw, self.k_blk_raw, self.prologue)

    def step(self) -> None:
        """One pass of the hot path over the batch: q/k norm + RoPE, block attention
        (two calls; q and k_blk are normalised in place)."""
        self.qk_norm_rope()
        self.attention()

    def step_fused(self) -> None:
        """One pass of the hot path as a single fused call (bf16)."""
        self.attention_fused()


class LayerPath:
    """The draft layer's attention block on the GPU: input norm + merged q/k/v
    projection of the block rows, the attention with the fused q/k norm +
    RoPE over [context; block], o_proj. The context rows come from
    ``DevicePath`` (packed store)."""

    def __init__(self, wl: Workload, li: LayerInputs, device: str = "cuda",
                 use_residual: bool = True):
        if wl.dtype != "bf16":
            raise ValueError("the layer path is bf16")
        self.wl, self.li = wl, li
        self.dp = DevicePath(wl, device)
        self.dp.prepare_context()
        t, h = wl.total_blk, li.hidden_size
        self.hidden = bits_to_device(li.hidden, device)
        self.residual_init = bits_to_device(li.residual, device) if use_residual else None
        self.residual = None if self.residual_init is None else self.residual_init.clone()
        self.in_norm_w = torch.from_numpy(np.ascontiguousarray(li.in_norm_w, np.float32)).to(device)
        self.w_qkv = bits_to_device(li.w_qkv, device)
        self.w_o = bits_to_device(li.w_o, device)
        bf = torch.bfloat16
        self.q = torch.empty((t, wl.hq, wl.dh), dtype=bf, device=device)
        self.k = torch.empty((t, wl.hkv, wl.dh), dtype=bf, device=device)
        self.v = torch.empty((t, wl.hkv, wl.dh), dtype=bf, device=device)
        self.o = torch.empty((t, h), dtype=bf, device=device)
        self.ws_qkv = B.alloc_workspace(
            B.dflash_block_qkv_workspace_size(t, h, wl.hq, wl.hkv, wl.dh), device)
        self.ws_o = B.alloc_workspace(B.dflash_o_proj_workspace_size(t, h, wl.hq * wl.dh), device)

    def reset_residual(self) -> None:
        if self.residual is not None:
            self.residual.copy_(self.residual_init)

    def qkv(self) -> None:
        B.dflash_block_qkv(self.hidden, self.residual, self.in_norm_w, self.w_qkv, self.wl.hq,
                           self.wl.hkv, self.wl.dh, self.wl.eps, self.q, self.k, self.v,
                           self.ws_qkv)

    def attention(self) -> None:
        dp = self.dp
        B.dflash_block_attention(dp.params, dp.cu_ctx, dp.cu_blk, self.q, self.k, self.v,
                                 dp.k_ctx if self.wl.total_ctx > 0 else None,
                                 dp.v_ctx if self.wl.total_ctx > 0 else None, dp.out, dp.ws,
                                 prologue=dp.prologue)

    def o_proj(self) -> None:
        B.dflash_o_proj(self.dp.out, self.w_o, self.o, self.ws_o)

    def step(self) -> None:
        self.qkv()
        self.attention()
        self.o_proj()


class DraftStep:
    """One propose step of a draft layer, every stage a library call on one
    stream with fixed buffers, so the whole step can be captured into a HIP
    graph and replayed with its inputs refreshed in place:

      dflash_prepare_inputs -> dflash_fc_combine (the target's tapped features
      of the verified rows) -> dflash_context_kv (their K/V at the prepared
      context positions) -> dflash_kv_scatter (into the paged store at the
      prepared slots) -> dflash_block_qkv (the block rows' hidden states) ->
      dflash_block_attention_paged (fused q/k norm + RoPE at the prepared block
      positions; the work split planned on the device from ctx_cu and
      query_start_loc) -> dflash_o_proj.

    Each request verifies ``rows_per_req`` rows per step; the block rows'
    hidden states (the embedding of the anchor + mask tokens, outside this
    library) are a fixed synthetic input. ``causal`` / ``window`` are the
    layer's mask flags (a sliding-window layer is causal with a window)."""

    def __init__(self, num_reqs: int, nqpr: int, rows_per_req: int, hidden: int = 256,
                 taps: int = 3, hq: int = 4, hkv: int = 2, dh: int = 128, pages_per_req: int = 16,
                 seed: int = 0, device: str = "cuda", eps: float = 1e-6, theta: float = 1e6,
                 causal: bool = False, window: int = 0):
        rng = np.random.default_rng(seed)
        self.r, self.nqpr, self.rows = num_reqs, nqpr, rows_per_req
        self.h, self.taps, self.hq, self.hkv, self.dh = hidden, taps, hq, hkv, dh
        self.eps = eps
        dev = device
        i32 = lambda a: torch.tensor(np.asarray(a, dtype=np.int32), device=dev)
        bits = lambda shape, s: bits_to_device(f32_to_bf16_bits(
            rng.standard_normal(shape, dtype=np.float32) * np.float32(s)), dev)
        f32w = lambda n: torch.from_numpy(bf16_bits_to_f32(f32_to_bf16_bits(
            rng.uniform(0.5, 1.5, n).astype(np.float32)))).to(dev)
        page = 16
        self.pages = num_reqs * pages_per_req + 3
        bt = rng.permutation(self.pages)[:num_reqs * pages_per_req].reshape(num_reqs, pages_per_req)
        self.block_table = i32(bt)
        ntgt = num_reqs * rows_per_req
        # inputs refreshed in place every step
        self.ins = {n: torch.zeros(ntgt if n == "target_positions" else
                                   (num_reqs + 1 if n == "target_query_start_loc" else num_reqs),
                                   dtype=torch.int32, device=dev)
                    for n in B.PREP_IN if n != "block_table"}
        self.ins["block_table"] = self.block_table
        self.ins["target_query_start_loc"].copy_(torch.arange(num_reqs + 1, dtype=torch.int32) * rows_per_req)
        self.ins["idx_mapping"].copy_(torch.arange(num_reqs, dtype=torch.int32))
        self.aux = torch.zeros((ntgt, hidden * taps), dtype=torch.float32, device=dev)
        sizes = dict(input_ids=num_reqs * nqpr, query_positions=num_reqs * nqpr,
                     query_start_loc=num_reqs + 1, seq_lens=num_reqs,
                     query_slot_mapping=num_reqs * nqpr, context_positions=ntgt,
                     context_slot_mapping=ntgt, sample_indices=num_reqs * (nqpr - 1),
                     sample_pos=num_reqs * (nqpr - 1), sample_idx_mapping=num_reqs * (nqpr - 1),
                     ctx_cu=num_reqs + 1)
        self.outs = {n: torch.zeros(sizes[n], dtype=torch.int32, device=dev) for n in B.PREP_OUT}
        self.prep = B.PrepareParams(num_reqs, num_reqs, num_reqs * nqpr, nqpr, nqpr - 1, page,
                                    pages_per_req, 1 << 20, 7, 0, num_reqs, ntgt)
        # weights (synthetic, bf16) and norm weights
        self.w_fc = bits((hidden, hidden * taps), 0.05)
        self.hnw, self.knw, self.qnw, self.in_norm_w = f32w(hidden), f32w(dh), f32w(dh), f32w(hidden)
        self.w_k, self.w_v = bits((hkv * dh, hidden), 0.05), bits((hkv * dh, hidden), 0.05)
        self.w_qkv = bits(((hq + 2 * hkv) * dh, hidden), 0.05)
        self.w_o = bits((hidden, hq * dh), 0.05)
        self.blk_hidden = bits((num_reqs * nqpr, hidden), 1.0)
        self.rope = torch.empty((1 << 14, dh // 2, 2), dtype=torch.float32, device=dev)
        B.dflash_rope_table(self.rope, 1 << 14, dh, theta)
        bf = torch.bfloat16
        self.k_pool = torch.zeros((self.pages, page, hkv, dh), dtype=bf, device=dev)
        self.v_pool = torch.zeros_like(self.k_pool)
        self.comb = torch.empty((ntgt, hidden), dtype=bf, device=dev)
        self.k_new = torch.empty((ntgt, hkv, dh), dtype=bf, device=dev)
        self.v_new = torch.empty_like(self.k_new)
        t = num_reqs * nqpr
        self.q = torch.empty((t, hq, dh), dtype=bf, device=dev)
        self.kb = torch.empty((t, hkv, dh), dtype=bf, device=dev)
        self.vb = torch.empty_like(self.kb)
        self.attn = torch.empty_like(self.q)
        self.o = torch.empty((t, hidden), dtype=bf, device=dev)
        self.params = B.make_block_attn_params(num_reqs, hq, hkv, dh, B.DFLASH_BF16,
                                               num_reqs * pages_per_req * page, t, nqpr, dh ** -0.5,
                                               causal=causal, window=window)
        self.pg = B.make_paged_ctx(self.block_table, self.pages)
        self.pro = B.make_qk_prologue(self.qnw, self.knw, self.outs["query_positions"], self.rope, eps)
        self.ws_fc = B.alloc_workspace(B.dflash_fc_combine_workspace_size(ntgt, hidden, taps), dev)
        self.ws_ckv = B.alloc_workspace(B.dflash_context_kv_workspace_size(ntgt, hidden, hkv, dh), dev)
        self.ws_qkv = B.alloc_workspace(B.dflash_block_qkv_workspace_size(t, hidden, hq, hkv, dh), dev)
        self.ws_attn = B.alloc_workspace(B.dflash_block_attention_paged_workspace_size(self.params), dev)
        self.ws_o = B.alloc_workspace(B.dflash_o_proj_workspace_size(t, hidden, hq * dh), dev)

    def set_step(self, positions, rejected, sampled, last_sampled, aux) -> None:
        """Refresh the step's inputs in place (host arrays)."""
        self.ins["target_positions"].copy_(torch.from_numpy(np.asarray(positions, np.int32)))
        self.ins["num_rejected"].copy_(torch.from_numpy(np.asarray(rejected, np.int32)))
        self.ins["num_sampled"].copy_(torch.from_numpy(np.asarray(sampled, np.int32)))
        self.ins["last_sampled"].copy_(torch.from_numpy(np.asarray(last_sampled, np.int32)))
        self.aux.copy_(torch.from_numpy(np.ascontiguousarray(aux, np.float32)))

    def run(self) -> None:
        o = self.outs
        B.dflash_prepare_inputs(self.prep, self.ins, o)
        B.dflash_fc_combine(self.aux, self.w_fc, self.comb, self.ws_fc)
        B.dflash_context_kv(self.comb, self.hnw, self.w_k, self.w_v, self.knw, o["context_positions"],
                            self.hkv, self.dh, self.eps, self.rope, self.k_new, self.v_new, self.ws_ckv)
        B.dflash_kv_scatter(self.k_new, self.v_new, o["context_slot_mapping"], self.k_pool, self.v_pool)
        B.dflash_block_qkv(self.blk_hidden, None, self.in_norm_w, self.w_qkv, self.hq, self.hkv,
                           self.dh, self.eps, self.q, self.kb, self.vb, self.ws_qkv)
        B.dflash_block_attention_paged(self.params, self.pg, o["ctx_cu"], o["query_start_loc"], self.q,
                                       self.kb, self.vb, self.k_pool, self.v_pool, self.attn,
                                       self.ws_attn, prologue=self.pro)
        B.dflash_o_proj(self.attn, self.w_o, self.o, self.ws_o)
