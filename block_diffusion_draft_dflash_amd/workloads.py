"""Seeded synthetic inputs for the DFlash block-attention path.

This module only draws and lays out inputs; it holds none of the method's
arithmetic. Both the HIP path and the CPU oracle are fed from it. Inputs are
drawn in float32 with ``numpy.random.default_rng(seed)`` and, for bf16
workloads, rounded to bfloat16 (round to nearest even) so that both sides see
exactly the same values.

Shapes follow the draft model's attention layer as the "qwen3_dflash.cpp"
page lays it out: block Q ``[T, Hq, Dh]``, block K/V ``[T, Hkv, Dh]``, packed
context K/V ``[sum C, Hkv, Dh]`` (the ``ContextKVDev`` record stores
``[C, Hkv*Dh]`` per layer), cumulative row counts per request, context rows at
positions ``0..C-1`` and the block (anchor + mask slots) at ``C..C+B-1``
(the propose step on the "runner.cpp" page).

Draw order is fixed: lengths, Q, K_blk, V_blk, K_ctx, V_ctx, q_norm, k_norm,
hidden_norm, hidden, W_k, W_v.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = [
    "Workload",
    "CONFIGS",
    "make_workload",
    "LayerInputs",
    "make_layer_inputs",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
]


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    bits = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        bits[nan] = 0x7FC0
    return bits


def bf16_bits_to_f32(bits):
    """Widen bfloat16 bit patterns to float32 exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


@dataclasses.dataclass
class Workload:
    """One synthetic batch. Floating arrays are float32 values; for bf16
    workloads they are exactly bf16-representable and ``*_bits`` hold the bits."""

    name: str
    dtype: str                 # "f32" or "bf16"
    num_reqs: int
    hq: int
    hkv: int
    dh: int
    ctx_lens: np.ndarray       # [R] int32
    blk_lens: np.ndarray       # [R] int32
    cu_ctx: np.ndarray         # [R+1] int32
    cu_blk: np.ndarray         # [R+1] int32
    ctx_positions: np.ndarray  # [sum C] int32, 0..C_r-1 per request
    blk_positions: np.ndarray  # [T] int32, C_r..C_r+B_r-1 per request
    q: np.ndarray              # [T, Hq, Dh] raw (before q-norm / RoPE)
    k_blk: np.ndarray          # [T, Hkv, Dh] raw
    v_blk: np.ndarray          # [T, Hkv, Dh]
    k_ctx: Optional[np.ndarray]  # [sum C, Hkv, Dh] raw (None when hidden is given)
    v_ctx: Optional[np.ndarray]  # [sum C, Hkv, Dh]     (None when hidden is given)
    q_norm_w: np.ndarray       # [Dh]
    k_norm_w: np.ndarray       # [Dh]
    causal: bool
    window: int
    eps: float
    theta: float
    hidden: Optional[np.ndarray] = None        # [sum C, H] bf16 bits (uint16)
    hidden_norm_w: Optional[np.ndarray] = None  # [H]
    w_k: Optional[np.ndarray] = None           # [Hkv*Dh, H] bf16 bits
    w_v: Optional[np.ndarray] = None           # [Hkv*Dh, H] bf16 bits

    @property
    def total_ctx(self) -> int:
        return int(self.cu_ctx[-1])

    @property
    def total_blk(self) -> int:
        return int(self.cu_blk[-1])

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.dh)

    @property
    def hidden_size(self) -> int:
        return 0 if self.hidden is None else int(self.hidden.shape[1])

    def visible_keys(self) -> np.ndarray:
        """Per request, the number of key rows some block query can see."""
        out = []
        for c, b in zip(self.ctx_lens.tolist(), self.blk_lens.tolist()):
            n = c + b
            if self.causal and self.window > 0:
                lo = max(0, c - self.window + 1)
                out.append(n - lo)
            else:
                out.append(n)
        return np.asarray(out, dtype=np.int64)


# name -> (config id, defaults). The ids give the seeds (1000 + id).
CONFIGS = {
    "tiny": dict(cid=1, num_reqs=1, ctx="fixed", ctx_len=64, blk=16, hq=4, hkv=2, dh=64,
                 dtype="f32", causal=False, window=0),
    "qwen3_8b_draft": dict(cid=2, num_reqs=8, ctx="uniform", ctx_lo=512, ctx_hi=2048, blk=16,
                           hq=32, hkv=8, dh=128, dtype="bf16", causal=False, window=0),
    "large_decode": dict(cid=3, num_reqs=64, ctx="loguniform", ctx_lo=128, ctx_hi=8192, blk=16,
                         hq=32, hkv=8, dh=128, dtype="bf16", causal=False, window=0),
    "swa": dict(cid=4, num_reqs=16, ctx="fixed", ctx_len=16384, blk=16, hq=32, hkv=8, dh=128,
                dtype="bf16", causal=True, window=4096),
    "ctx_kv": dict(cid=5, num_reqs=4, ctx="fixed", ctx_len=32768, blk=16, hq=32, hkv=8, dh=128,
                   dtype="bf16", causal=False, window=0, hidden=4096),
}


def _draw(rng, shape, dtype, kind="normal", lo=0.0, hi=1.0, std=1.0):
    if kind == "normal":
        x = rng.standard_normal(size=shape, dtype=np.float32)
        if std != 1.0:
            x = (x * np.float32(std)).astype(np.float32)
    else:
        x = rng.uniform(lo, hi, size=shape).astype(np.float32)
    if dtype == "bf16":
        return bf16_bits_to_f32(f32_to_bf16_bits(x)).reshape(shape)
    return x


def make_workload(name: str, seed: Optional[int] = None, **over) -> Workload:
    """Draw one batch of the named configuration.

    Keyword overrides replace configuration fields (e.g. ``num_reqs``,
    ``ctx_len``, ``ctx_lo``/``ctx_hi``, ``blk``, ``window``, ``hidden``), so
    tests can draw the same kind of input at sizes the oracle finishes quickly.
    ``ctx_lens`` may be given explicitly as a list.
    """
    cfg = dict(CONFIGS[name])
    cfg.update(over)
    if seed is None:
        seed = 1000 + cfg["cid"]
    rng = np.random.default_rng(seed)
    r = int(cfg["num_reqs"])
    dt = cfg["dtype"]
    hq, hkv, dh = int(cfg["hq"]), int(cfg["hkv"]), int(cfg["dh"])

    # lengths
    if "ctx_lens" in over:
        ctx = np.asarray(over["ctx_lens"], dtype=np.int64)
        r = len(ctx)
    elif cfg["ctx"] == "fixed":
        ctx = np.full(r, int(cfg["ctx_len"]), dtype=np.int64)
    elif cfg["ctx"] == "uniform":
        ctx = rng.integers(int(cfg["ctx_lo"]), int(cfg["ctx_hi"]) + 1, size=r)
    elif cfg["ctx"] == "loguniform":
        u = rng.uniform(math.log(cfg["ctx_lo"]), math.log(cfg["ctx_hi"]), size=r)
        ctx = np.rint(np.exp(u)).astype(np.int64)
    else:
        raise ValueError(cfg["ctx"])
    if "blk_lens" in over:
        blk = np.asarray(over["blk_lens"], dtype=np.int64)
    else:
        blk = np.full(r, int(cfg["blk"]), dtype=np.int64)
    cu_ctx = np.concatenate([[0], np.cumsum(ctx)]).astype(np.int32)
    cu_blk = np.concatenate([[0], np.cumsum(blk)]).astype(np.int32)
    c_tot, t_tot = int(cu_ctx[-1]), int(cu_blk[-1])
    ctx_pos = np.concatenate([np.arange(c, dtype=np.int32) for c in ctx.tolist()] or
                             [np.zeros(0, np.int32)]).astype(np.int32)
    blk_pos = np.concatenate([np.arange(c, c + b, dtype=np.int32)
                              for c, b in zip(ctx.tolist(), blk.tolist())] or
                             [np.zeros(0, np.int32)]).astype(np.int32)

    q = _draw(rng, (t_tot, hq, dh), dt)
    k_blk = _draw(rng, (t_tot, hkv, dh), dt)
    v_blk = _draw(rng, (t_tot, hkv, dh), dt)
    hidden_size = int(cfg.get("hidden", 0) or 0)
    if hidden_size:
        k_ctx = v_ctx = None
    else:
        k_ctx = _draw(rng, (c_tot, hkv, dh), dt)
        v_ctx = _draw(rng, (c_tot, hkv, dh), dt)
    q_norm_w = _draw(rng, (dh,), "bf16", "uniform", 0.5, 1.5)
    k_norm_w = _draw(rng, (dh,), "bf16", "uniform", 0.5, 1.5)
    wl = Workload(
        name=name, dtype=dt, num_reqs=r, hq=hq, hkv=hkv, dh=dh,
        ctx_lens=ctx.astype(np.int32), blk_lens=blk.astype(np.int32),
        cu_ctx=cu_ctx, cu_blk=cu_blk, ctx_positions=ctx_pos, blk_positions=blk_pos,
        q=q, k_blk=k_blk, v_blk=v_blk, k_ctx=k_ctx, v_ctx=v_ctx,
        q_norm_w=q_norm_w, k_norm_w=k_norm_w,
        causal=bool(cfg["causal"]), window=int(cfg["window"]),
        eps=float(cfg.get("eps", 1e-6)), theta=float(cfg.get("theta", 1e6)),
    )
    if hidden_size:
        wl.hidden_norm_w = _draw(rng, (hidden_size,), "bf16", "uniform", 0.5, 1.5)
        # Draw the hidden states in row blocks to bound peak host memory.
        bits = np.empty((c_tot, hidden_size), dtype=np.uint16)
        step = 8192
        for s in range(0, c_tot, step):
            e = min(c_tot, s + step)
            bits[s:e] = f32_to_bf16_bits(
                rng.standard_normal(size=(e - s, hidden_size), dtype=np.float32))
        wl.hidden = bits
        kdim = hkv * dh
        wl.w_k = f32_to_bf16_bits(rng.standard_normal((kdim, hidden_size), dtype=np.float32)
                                  * np.float32(0.02))
        wl.w_v = f32_to_bf16_bits(rng.standard_normal((kdim, hidden_size), dtype=np.float32)
                                  * np.float32(0.02))
    return wl


@dataclasses.dataclass
class LayerInputs:
    """Inputs of the draft layer around the attention for a workload's block
    rows (bf16 bits as uint16; float arrays exactly bf16-representable)."""

    hidden_size: int
    hidden: np.ndarray        # [T, H] bf16 bits: the block rows' hidden states
    residual: np.ndarray      # [T, H] bf16 bits: the residual stream before the layer
    in_norm_w: np.ndarray     # [H] input_layernorm weight
    w_qkv: np.ndarray         # [(Hq + 2 Hkv) Dh, H] bf16 bits: rows q heads | k heads | v heads
    w_o: np.ndarray           # [H, Hq Dh] bf16 bits


def make_layer_inputs(wl: Workload, hidden_size: int, seed: Optional[int] = None) -> LayerInputs:
    """Draw the layer inputs for ``wl``'s block rows from a generator of their
    own (the workload's own draws are unchanged): hidden and residual ~N(0, 1),
    the norm weight ~U(0.5, 1.5), the projection weights ~N(0, 0.02), in that
    order, all rounded to bf16."""
    rng = np.random.default_rng(seed if seed is not None else 5000 + hidden_size + wl.total_blk)
    t = wl.total_blk
    n_qkv = (wl.hq + 2 * wl.hkv) * wl.dh
    hid = f32_to_bf16_bits(rng.standard_normal((t, hidden_size), dtype=np.float32))
    res = f32_to_bf16_bits(rng.standard_normal((t, hidden_size), dtype=np.float32))
    w_in = _draw(rng, (hidden_size,), "bf16", "uniform", 0.5, 1.5)
    w_qkv = f32_to_bf16_bits(rng.standard_normal((n_qkv, hidden_size), dtype=np.float32)
                             * np.float32(0.02))
    w_o = f32_to_bf16_bits(rng.standard_normal((hidden_size, wl.hq * wl.dh), dtype=np.float32)
                           * np.float32(0.02))
    return LayerInputs(hidden_size, hid, res, w_in, w_qkv, w_o)
