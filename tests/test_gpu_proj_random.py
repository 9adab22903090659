"""Seeded random shapes through the projection entry points and the standalone
q/k norm + RoPE, each against the fp64 oracle at the bounds the fixed-shape
tests derive (test_gpu_layer.py for dflash_block_qkv and dflash_o_proj,
test_gpu_propose.py for dflash_fc_combine and dflash_context_kv,
test_gpu_parity.py's one-rounding bound for dflash_qk_norm_rope).

Row counts, hidden sizes, head geometries and the residual are drawn per case,
so the planner's branches (128- and 64-wide column tiles, uneven and
power-of-two K splits, a single slice, the few-row and the large-row context
forms, partial row tiles) all meet the oracle. The kind of call cycles with
the case number; DFLASH_RANDOM_CASES=N runs the first N seeds (20 by default).
"""
import os

import numpy as np
import pytest
import torch

from block_diffusion_draft_dflash_amd import binding as B
from block_diffusion_draft_dflash_amd.pipeline import bits_to_device, to_host_f64
from block_diffusion_draft_dflash_amd.workloads import bf16_bits_to_f32, f32_to_bf16_bits
from test_gpu_layer import _check_bound
from test_gpu_propose import _context_kv_vs_oracle

pytestmark = pytest.mark.gpu

N_CASES = int(os.environ.get("DFLASH_RANDOM_CASES", "20"))
KINDS = ("block_qkv", "o_proj", "fc_combine", "context_kv", "qk_norm_rope")


def _bits(rng, shape, scale):
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(scale))


def _f(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def _block_qkv(rng, tag):
    from oracle import dflash_oracle as O
    t = int(rng.integers(1, 301))
    h = 64 * int(rng.integers(1, 65))
    hkv = int(rng.choice([1, 2, 4, 8]))
    hq = hkv * int(rng.choice([1, 2, 4]))
    dh = int(rng.choice([64, 128]))
    use_res = bool(rng.random() < 0.7)
    print(f"case {tag}: T={t} H={h} Hq={hq} Hkv={hkv} Dh={dh} residual={use_res}", flush=True)
    n = (hq + 2 * hkv) * dh
    hid_bits, res_bits, w_bits = _bits(rng, (t, h), 1.0), _bits(rng, (t, h), 1.0), _bits(rng, (n, h), 0.02)
    nw = bf16_bits_to_f32(f32_to_bf16_bits(rng.uniform(0.5, 1.5, h).astype(np.float32)))
    dev = "cuda"
    res = bits_to_device(res_bits, dev) if use_res else None
    q = torch.full((t, hq, dh), float("nan"), dtype=torch.bfloat16, device=dev)
    k = torch.full((t, hkv, dh), float("nan"), dtype=torch.bfloat16, device=dev)
    v = torch.full((t, hkv, dh), float("nan"), dtype=torch.bfloat16, device=dev)
    ws = B.alloc_workspace(B.dflash_block_qkv_workspace_size(t, h, hq, hkv, dh), dev)
    B.dflash_block_qkv(bits_to_device(hid_bits, dev), res, torch.from_numpy(nw).to(dev),
                       bits_to_device(w_bits, dev), hq, hkv, dh, 1e-6, q, k, v, ws)
    torch.cuda.synchronize()
    _, normed = O.residual_rms_norm(_f(hid_bits), _f(res_bits) if use_res else None, nw, 1e-6)
    qo, ko, vo = O.block_qkv(normed, _f(w_bits), hq, hkv, dh)
    absprod = np.abs(normed) @ np.abs(_f(w_bits)).T
    qd, kd = hq * dh, hkv * dh
    for name, g, o, ap in (("q", q, qo, absprod[:, :qd]), ("k", k, ko, absprod[:, qd:qd + kd]),
                           ("v", v, vo, absprod[:, qd + kd:])):
        _check_bound(f"{tag} {name}", to_host_f64(g).reshape(t, -1), o.reshape(t, -1), ap,
                     2.0 ** -7, 2.0 ** -8)


def _o_proj(rng, tag):
    from oracle import dflash_oracle as O
    t = int(rng.integers(1, 601))
    h = 64 * int(rng.integers(1, 65))
    in_dim = 64 * int(rng.integers(1, 65))
    print(f"case {tag}: T={t} H={h} in_dim={in_dim}", flush=True)
    a_bits, w_bits = _bits(rng, (t, in_dim), 0.3), _bits(rng, (h, in_dim), 0.02)
    dev = "cuda"
    out = torch.full((t, h), float("nan"), dtype=torch.bfloat16, device=dev)
    ws = B.alloc_workspace(B.dflash_o_proj_workspace_size(t, h, in_dim), dev)
    B.dflash_o_proj(bits_to_device(a_bits, dev), bits_to_device(w_bits, dev), out, ws)
    torch.cuda.synchronize()
    a, w = _f(a_bits), _f(w_bits)
    _check_bound(f"{tag} o_proj", to_host_f64(out), O.output_projection(a, w), np.abs(a) @ np.abs(w).T,
                 2.0 ** -11, 2.0 ** -8)


def _fc_combine(rng, tag):
    from oracle import dflash_oracle as O
    t = int(rng.integers(1, 301))
    h = 64 * int(rng.integers(1, 33))
    taps = int(rng.integers(1, min(6, 8192 // h) + 1))
    print(f"case {tag}: T={t} H={h} taps={taps}", flush=True)
    aux = rng.standard_normal((t, h * taps), dtype=np.float32) * np.float32(2.0)
    w_bits = _bits(rng, (h, h * taps), 0.02)
    out = torch.full((t, h), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = B.alloc_workspace(B.dflash_fc_combine_workspace_size(t, h, taps))
    B.dflash_fc_combine(torch.from_numpy(aux).cuda(), bits_to_device(w_bits), out, ws)
    torch.cuda.synchronize()
    a, w = O.bf16_round(aux), _f(w_bits)
    _check_bound(f"{tag} fc", to_host_f64(out), O.fc_combine(a, w), np.abs(a) @ np.abs(w).T,
                 2.0 ** -11, 2.0 ** -8)


def _context_kv(rng, tag):
    rows = int(rng.integers(1, 1101))
    hkv = int(rng.choice([2, 4, 8]))
    h = 64 * int(rng.integers(1, 33))
    print(f"case {tag}: rows={rows} Hkv={hkv} H={h}", flush=True)
    _context_kv_vs_oracle(rows, hkv, h)


def _qk_norm_rope(rng, tag):
    # head counts that leave partial chunks of the kernel's 8-head lane groups,
    # the K-only form, both dtypes, and positions past either end of the table
    # (the call clamps them into it)
    from oracle import dflash_oracle as O
    t = int(rng.integers(1, 3001))
    hkv = int(rng.choice([1, 2, 3, 4, 8, 16]))
    hq = hkv * int(rng.choice([1, 2, 4, 5, 8])) if rng.random() < 0.8 else 0
    dh = int(rng.choice([64, 128]))
    f32 = bool(rng.random() < 0.3)
    max_pos = int(rng.integers(1, 50001))
    print(f"case {tag}: T={t} Hq={hq} Hkv={hkv} Dh={dh} {'f32' if f32 else 'bf16'} max_pos={max_pos}",
          flush=True)
    dev = "cuda"
    pos = rng.integers(-50, max_pos + 50, size=t).astype(np.int32)
    rnd = (lambda x: x.astype(np.float32)) if f32 else \
        (lambda x: bf16_bits_to_f32(f32_to_bf16_bits(x.astype(np.float32))))
    k = rnd(rng.standard_normal((t, hkv, dh)))
    q = rnd(rng.standard_normal((t, hq, dh))) if hq else None
    kw = bf16_bits_to_f32(f32_to_bf16_bits(rng.uniform(0.5, 1.5, dh).astype(np.float32)))
    qw = bf16_bits_to_f32(f32_to_bf16_bits(rng.uniform(0.5, 1.5, dh).astype(np.float32)))
    dt = torch.float32 if f32 else torch.bfloat16
    kd = torch.from_numpy(k).to(dev).to(dt)
    qd = torch.from_numpy(q).to(dev).to(dt) if hq else None
    table = torch.empty((max_pos, dh // 2, 2), dtype=torch.float32, device=dev)
    B.dflash_rope_table(table, max_pos, dh, 1e6)
    B.dflash_qk_norm_rope(qd, kd, torch.from_numpy(qw).to(dev) if hq else None, torch.from_numpy(kw).to(dev),
                          torch.from_numpy(pos).to(dev), 1e-6, table)
    torch.cuda.synchronize()
    eff = np.clip(pos, 0, max_pos - 1)
    qo, ko = O.qk_norm_rope(q.astype(np.float64) if hq else None, k.astype(np.float64), qw, kw, eff, 1e-6, 1e6)
    rel = 1e-6 if f32 else 2.0 ** -7
    for name, g, o in (("k", kd, ko), ("q", qd, qo)):
        if g is None:
            continue
        err = np.abs(to_host_f64(g) - o)
        print(f"[{tag} {name}] max abs {err.max():.3e}", flush=True)
        assert (err <= rel * np.abs(o) + 1e-5).all(), f"{tag} {name}: beyond the one-rounding bound"


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_projection_shape(i):
    rng = np.random.default_rng(9100 + i)
    kind = KINDS[i % len(KINDS)]
    fn = {"block_qkv": _block_qkv, "o_proj": _o_proj, "fc_combine": _fc_combine,
          "context_kv": _context_kv, "qk_norm_rope": _qk_norm_rope}[kind]
    fn(rng, f"random {i} {kind}")
