"""Pins of the fp64 oracle to things other than itself (CPU only).

Each pin checks the oracle against a closed form, an invariant the mathematics
fixes, an independent library routine (torch fp64 CPU ops) or a brute-force
second formulation on tiny inputs. ``test_pins_catch_planted_mistakes`` plants
plausible mistakes in the oracle (a dropped term, a wrong sign, a wrong index,
a transposed operand) and checks that some pin fails for each.

The pages print no worked numeric example, so there are no printed values to
pin against (no fixture under tests/golden/ comes from the pages).
"""
import math
import types

import numpy as np
import pytest
import torch

import oracle
from oracle import dflash_oracle as O

RNG = np.random.default_rng(12345)


def _ns(**over):
    """The oracle's functions as a namespace, optionally with some replaced."""
    base = dict(
        rms_norm=O.rms_norm,
        rope_neox=O.rope_neox,
        qk_norm_rope=O.qk_norm_rope,
        context_projection=O.context_projection,
        context_kv=O.context_kv,
        attention_visibility=O.attention_visibility,
        block_attention=O.block_attention,
    )
    base.update(over)
    return types.SimpleNamespace(**base)


# ----------------------------------------------------------------------------- RMSNorm pins

def pin_rms_norm_library(X):
    x = RNG.standard_normal((7, 33))
    w = RNG.uniform(0.5, 1.5, 33)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (33,), torch.from_numpy(w), eps=1e-6)
    np.testing.assert_allclose(X.rms_norm(x, w, 1e-6), ref.numpy(), rtol=1e-13, atol=1e-13)


def pin_rms_norm_closed_form(X):
    # Unit weight: the output's mean square is ms / (ms + eps) exactly.
    x = RNG.standard_normal((5, 64)) * 0.01
    eps = 1e-4
    y = X.rms_norm(x, np.ones(64), eps)
    ms = np.mean(x * x, axis=1)
    np.testing.assert_allclose(np.mean(y * y, axis=1), ms / (ms + eps), rtol=1e-12)
    # Weight multiplies element-wise; a single constant row c gives c / sqrt(c^2 + eps).
    c = 0.3
    y = X.rms_norm(np.full((1, 4), c), np.array([1.0, 2.0, 0.5, 1.0]), 1e-2)
    np.testing.assert_allclose(y[0], np.array([1.0, 2.0, 0.5, 1.0]) * c / math.sqrt(c * c + 1e-2),
                               rtol=1e-14)


# ----------------------------------------------------------------------------- RoPE pins

def pin_rope_complex_form(X):
    # NeoX rotate-half == complex multiply of (x_i + i x_{i+D/2}) by exp(i p f_i).
    t, h, d, theta = 6, 3, 16, 1e4
    x = RNG.standard_normal((t, h, d))
    pos = RNG.integers(0, 5000, t)
    f = theta ** (-np.arange(d // 2) * 2.0 / d)
    z = (x[..., : d // 2] + 1j * x[..., d // 2:]) * np.exp(1j * pos[:, None, None] * f[None, None, :])
    ref = np.concatenate([z.real, z.imag], axis=-1)
    np.testing.assert_allclose(X.rope_neox(x, pos, theta), ref, rtol=1e-12, atol=1e-12)


def pin_rope_hand_case(X):
    # Dh = 4, theta = 100: inverse frequencies 1 and 0.1; position 3.
    x = np.array([[[1.0, 2.0, 3.0, 4.0]]])
    y = X.rope_neox(x, np.array([3]), 100.0)[0, 0]
    a0, a1 = 3.0, 0.3
    ref = [1 * math.cos(a0) - 3 * math.sin(a0), 2 * math.cos(a1) - 4 * math.sin(a1),
           3 * math.cos(a0) + 1 * math.sin(a0), 4 * math.cos(a1) + 2 * math.sin(a1)]
    np.testing.assert_allclose(y, ref, rtol=1e-14, atol=1e-14)


def pin_rope_invariants(X):
    t, d, theta = 9, 64, 1e6
    x = RNG.standard_normal((t, 2, d))
    # position 0 is the identity
    np.testing.assert_allclose(X.rope_neox(x, np.zeros(t, int), theta), x, rtol=0, atol=0)
    # norm preserved
    pos = RNG.integers(0, 40000, t)
    y = X.rope_neox(x, pos, theta)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    # <R(q,p), R(k,p')> depends only on p - p'
    q = RNG.standard_normal((1, 1, d))
    k = RNG.standard_normal((1, 1, d))
    dots = []
    for p in (0, 17, 1000, 33000):
        rq = X.rope_neox(q, np.array([p + 5]), theta)
        rk = X.rope_neox(k, np.array([p]), theta)
        dots.append(float(np.sum(rq * rk)))
    np.testing.assert_allclose(dots, dots[0], rtol=1e-9)
    # element 0 pairs with element Dh/2 (rotate-half), nothing else moves
    e = np.zeros((1, 1, d))
    e[0, 0, 0] = 1.0
    y = X.rope_neox(e, np.array([7]), theta)[0, 0]
    nz = np.flatnonzero(np.abs(y) > 1e-15)
    assert nz.tolist() == [0, d // 2]
    np.testing.assert_allclose([y[0], y[d // 2]], [math.cos(7.0), math.sin(7.0)], rtol=1e-14)


def pin_qk_norm_then_rope(X):
    # norm first, rope second: with unit weights the rotated head keeps the
    # normed RMS; q and k rows use the same positions.
    t, d = 5, 32
    q = RNG.standard_normal((t, 4, d)) * 3.0
    k = RNG.standard_normal((t, 2, d)) * 0.2
    pos = np.arange(t) * 11
    wq = RNG.uniform(0.5, 1.5, d)
    wk = RNG.uniform(0.5, 1.5, d)
    qh, kh = X.qk_norm_rope(q, k, wq, wk, pos, 1e-6, 1e6)
    ref_q = X.rope_neox(torch.nn.functional.rms_norm(torch.from_numpy(q), (d,),
                                                     torch.from_numpy(wq), eps=1e-6).numpy(), pos, 1e6)
    np.testing.assert_allclose(qh, ref_q, rtol=1e-12, atol=1e-12)
    qu, ku = X.qk_norm_rope(q, k, np.ones(d), np.ones(d), pos, 0.0, 1e6)
    np.testing.assert_allclose(np.mean(ku * ku, axis=-1), 1.0, rtol=1e-12)
    np.testing.assert_allclose(np.mean(qu * qu, axis=-1), 1.0, rtol=1e-12)
    none_q, k_only = X.qk_norm_rope(None, k, None, wk, pos, 1e-6, 1e6)
    assert none_q is None
    np.testing.assert_allclose(k_only, kh, rtol=0, atol=0)


# ----------------------------------------------------------------------------- projection pins

def pin_projection_library(X):
    c, hsz, kdim = 9, 48, 16
    h = RNG.standard_normal((c, hsz))
    wn = RNG.uniform(0.5, 1.5, hsz)
    wk = RNG.standard_normal((kdim, hsz)) * 0.02
    wv = RNG.standard_normal((kdim, hsz)) * 0.02
    kr, v = X.context_projection(h, wn, wk, wv, 1e-6)
    th = torch.nn.functional.rms_norm(torch.from_numpy(h), (hsz,), torch.from_numpy(wn), eps=1e-6)
    np.testing.assert_allclose(kr, torch.nn.functional.linear(th, torch.from_numpy(wk)).numpy(),
                               rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(v, torch.nn.functional.linear(th, torch.from_numpy(wv)).numpy(),
                               rtol=1e-12, atol=1e-14)


def pin_context_kv_structure(X):
    # chunked == whole (rows are independent), V raw, K normed then rotated per head.
    c, hsz, hkv, d = 12, 40, 2, 8
    h = RNG.standard_normal((c, hsz))
    wn = RNG.uniform(0.5, 1.5, hsz)
    wk = RNG.standard_normal((hkv * d, hsz)) * 0.02
    wv = RNG.standard_normal((hkv * d, hsz)) * 0.02
    wkn = RNG.uniform(0.5, 1.5, d)
    pos = np.arange(c)
    k, v = X.context_kv(h, wn, wk, wv, wkn, pos, hkv, d, 1e-6, 1e6)
    k1, v1 = X.context_kv(h[:5], wn, wk, wv, wkn, pos[:5], hkv, d, 1e-6, 1e6)
    k2, v2 = X.context_kv(h[5:], wn, wk, wv, wkn, pos[5:], hkv, d, 1e-6, 1e6)
    np.testing.assert_allclose(np.concatenate([k1, k2]), k, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(np.concatenate([v1, v2]), v, rtol=1e-13, atol=1e-15)
    # torch composition of the same steps
    th = torch.nn.functional.rms_norm(torch.from_numpy(h), (hsz,), torch.from_numpy(wn), eps=1e-6)
    tk = torch.nn.functional.linear(th, torch.from_numpy(wk)).reshape(c, hkv, d)
    tv = torch.nn.functional.linear(th, torch.from_numpy(wv)).reshape(c, hkv, d)
    tkn = torch.nn.functional.rms_norm(tk, (d,), torch.from_numpy(wkn), eps=1e-6).numpy()
    f = 1e6 ** (-np.arange(d // 2) * 2.0 / d)
    z = (tkn[..., : d // 2] + 1j * tkn[..., d // 2:]) * np.exp(1j * pos[:, None, None] * f)
    np.testing.assert_allclose(k, np.concatenate([z.real, z.imag], -1), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(v, tv.numpy(), rtol=1e-12, atol=1e-15)
    # V per head in order: head g of V is rows g*d..(g+1)*d of the V weight.
    np.testing.assert_allclose(v[:, 1, :], (th.numpy() @ wv[d:2 * d].T), rtol=1e-12, atol=1e-15)


# ----------------------------------------------------------------------------- attention pins

def _rand_batch(ctx_lens, blk_lens, hq, hkv, d, seed):
    rng = np.random.default_rng(seed)
    cu_c = np.concatenate([[0], np.cumsum(ctx_lens)]).astype(np.int64)
    cu_b = np.concatenate([[0], np.cumsum(blk_lens)]).astype(np.int64)
    q = rng.standard_normal((cu_b[-1], hq, d))
    kb = rng.standard_normal((cu_b[-1], hkv, d))
    vb = rng.standard_normal((cu_b[-1], hkv, d))
    kc = rng.standard_normal((cu_c[-1], hkv, d))
    vc = rng.standard_normal((cu_c[-1], hkv, d))
    return q, kb, vb, kc, vc, cu_c, cu_b


def _brute(q, kb, vb, kc, vc, cu_c, cu_b, scale, causal, window):
    """Second formulation: explicit loops, explicit mask test, exp without max shift."""
    t, hq, d = q.shape
    hkv = kb.shape[1]
    out = np.zeros_like(q)
    for r in range(len(cu_b) - 1):
        cl = int(cu_c[r + 1] - cu_c[r])
        for b in range(int(cu_b[r + 1] - cu_b[r])):
            row = int(cu_b[r]) + b
            qi = cl + b  # index of this query in [context; block]
            for h in range(hq):
                g = h * hkv // hq
                ws, acc = [], [[] for _ in range(d)]
                for j in range(cl + int(cu_b[r + 1] - cu_b[r])):
                    if causal and (j > qi or (window > 0 and qi - j >= window)):
                        continue
                    kr = kc[int(cu_c[r]) + j, g] if j < cl else kb[int(cu_b[r]) + j - cl, g]
                    vr = vc[int(cu_c[r]) + j, g] if j < cl else vb[int(cu_b[r]) + j - cl, g]
                    s = math.fsum(float(a) * float(c) for a, c in zip(q[row, h], kr)) * scale
                    e = math.exp(s)
                    ws.append(e)
                    for i in range(d):
                        acc[i].append(e * float(vr[i]))
                z = math.fsum(ws)
                for i in range(d):
                    out[row, h, i] = math.fsum(acc[i]) / z
    return out


def pin_attention_brute_force(X):
    for causal, window in ((False, 0), (True, 0), (True, 5)):
        args = _rand_batch([7, 0, 12], [4, 3, 2], 4, 2, 8, 7)
        s = 1 / math.sqrt(8)
        got = X.block_attention(*args, s, causal, window)
        ref = _brute(*args, s, causal, window)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def pin_attention_library(X):
    # torch SDPA (fp64, CPU, explicit boolean mask, GQA by repeated kv heads).
    q, kb, vb, kc, vc, cu_c, cu_b = _rand_batch([30, 3], [6, 5], 8, 2, 16, 8)
    for causal, window in ((False, 0), (True, 0), (True, 9)):
        got = X.block_attention(q, kb, vb, kc, vc, cu_c, cu_b, 0.37, causal, window)
        for r in range(2):
            c0, c1, b0, b1 = cu_c[r], cu_c[r + 1], cu_b[r], cu_b[r + 1]
            n, bl = c1 - c0 + b1 - b0, b1 - b0
            keys = torch.from_numpy(np.concatenate([kc[c0:c1], kb[b0:b1]])).permute(1, 0, 2)
            vals = torch.from_numpy(np.concatenate([vc[c0:c1], vb[b0:b1]])).permute(1, 0, 2)
            qq = torch.from_numpy(q[b0:b1]).permute(1, 0, 2)
            qi = torch.arange(bl).reshape(-1, 1) + (c1 - c0)
            kj = torch.arange(n).reshape(1, -1)
            mask = torch.ones(bl, n, dtype=torch.bool)
            if causal:
                mask = kj <= qi
                if window > 0:
                    mask &= (qi - kj) < window
            ref = torch.nn.functional.scaled_dot_product_attention(
                qq, keys.contiguous(), vals.contiguous(), attn_mask=mask, scale=0.37,
                enable_gqa=True)
            np.testing.assert_allclose(got[b0:b1], ref.permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-12)


def pin_attention_closed_forms(X):
    q, kb, vb, kc, vc, cu_c, cu_b = _rand_batch([10, 4], [5, 3], 4, 2, 8, 9)
    # softmax rows sum to one: V == 1 gives output 1.
    got = X.block_attention(q, kb, np.ones_like(vb), kc, np.ones_like(vc), cu_c, cu_b, 0.5)
    np.testing.assert_allclose(got, 1.0, rtol=0, atol=1e-14)
    # one visible key (causal, window 1): output is the row's own V.
    got = X.block_attention(q, kb, vb, kc, vc, cu_c, cu_b, 0.5, True, 1)
    g = np.arange(4) * 2 // 4
    np.testing.assert_allclose(got, vb[:, g, :], rtol=0, atol=0)
    # empty context, one block row: output is that row's V.
    a = _rand_batch([0], [1], 4, 2, 8, 3)
    got = X.block_attention(*a, 0.9)
    np.testing.assert_allclose(got[0], a[2][0, g, :], rtol=0, atol=0)
    # all keys equal: output is the plain mean of the visible values.
    kc2 = np.broadcast_to(kc[:1], kc.shape).copy()
    kb2 = np.broadcast_to(kc[:1], kb.shape).copy()
    got = X.block_attention(q, kb2, vb, kc2, vc, cu_c, cu_b, 0.5)
    for r in range(2):
        vals = np.concatenate([vc[cu_c[r]:cu_c[r + 1]], vb[cu_b[r]:cu_b[r + 1]]])
        np.testing.assert_allclose(got[cu_b[r]:cu_b[r + 1]],
                                   np.broadcast_to(vals.mean(0)[g], got[cu_b[r]:cu_b[r + 1]].shape),
                                   rtol=1e-13, atol=1e-14)
    # causal, query b of a request sees C + b + 1 keys: with equal keys the
    # output is the mean of exactly those.
    got = X.block_attention(q, kb2, vb, kc2, vc, cu_c, cu_b, 0.5, True, 0)
    vals = np.concatenate([vc[0:10], vb[0:5]])
    for b in range(5):
        np.testing.assert_allclose(got[b], vals[: 10 + b + 1].mean(0)[g], rtol=1e-13, atol=1e-14)
    # window W >= C + B reduces to plain causal.
    np.testing.assert_allclose(X.block_attention(q, kb, vb, kc, vc, cu_c, cu_b, 0.5, True, 100),
                               X.block_attention(q, kb, vb, kc, vc, cu_c, cu_b, 0.5, True, 0),
                               rtol=0, atol=0)


def pin_attention_permutations(X):
    q, kb, vb, kc, vc, cu_c, cu_b = _rand_batch([9], [6], 4, 2, 8, 10)
    base = X.block_attention(q, kb, vb, kc, vc, cu_c, cu_b, 0.4)
    # block-query permutation equivariance (bidirectional)
    p = np.array([3, 0, 5, 1, 4, 2])
    np.testing.assert_allclose(X.block_attention(q[p], kb, vb, kc, vc, cu_c, cu_b, 0.4), base[p],
                               rtol=1e-13, atol=1e-14)
    # joint permutation of block (K, V) pairs, and of context pairs
    np.testing.assert_allclose(X.block_attention(q, kb[p], vb[p], kc, vc, cu_c, cu_b, 0.4), base,
                               rtol=1e-13, atol=1e-14)
    pc = RNG.permutation(9)
    np.testing.assert_allclose(X.block_attention(q, kb, vb, kc[pc], vc[pc], cu_c, cu_b, 0.4), base,
                               rtol=1e-13, atol=1e-14)
    # GQA: q-head h reads kv-head h // (Hq/Hkv)
    for h in range(4):
        g = h // 2
        one = X.block_attention(q[:, h:h + 1], kb[:, g:g + 1], vb[:, g:g + 1], kc[:, g:g + 1],
                                vc[:, g:g + 1], cu_c, cu_b, 0.4)
        np.testing.assert_allclose(base[:, h:h + 1], one, rtol=0, atol=0)
    # scale -> 0: mean of all values
    got = X.block_attention(q, kb, vb, kc, vc, cu_c, cu_b, 0.0)
    np.testing.assert_allclose(got, np.broadcast_to(np.concatenate([vc, vb]).mean(0)[[0, 0, 1, 1]],
                                                    got.shape), rtol=1e-13, atol=1e-14)


def pin_requests_independent(X):
    # A packed batch equals each request run alone.
    q, kb, vb, kc, vc, cu_c, cu_b = _rand_batch([5, 11, 0], [3, 4, 2], 4, 2, 8, 11)
    got = X.block_attention(q, kb, vb, kc, vc, cu_c, cu_b, 0.6, True, 6)
    for r in range(3):
        c0, c1, b0, b1 = cu_c[r], cu_c[r + 1], cu_b[r], cu_b[r + 1]
        one = X.block_attention(q[b0:b1], kb[b0:b1], vb[b0:b1], kc[c0:c1], vc[c0:c1],
                                [0, c1 - c0], [0, b1 - b0], 0.6, True, 6)
        np.testing.assert_allclose(got[b0:b1], one, rtol=0, atol=0)


def pin_visibility(X):
    v = X.attention_visibility(4, 3, True, 3)
    ref = np.array([[0, 0, 1, 1, 1, 0, 0],
                    [0, 0, 0, 1, 1, 1, 0],
                    [0, 0, 0, 0, 1, 1, 1]], dtype=bool)
    assert (v == ref).all()
    assert X.attention_visibility(4, 3, False, 0).all()
    with pytest.raises(ValueError):
        X.attention_visibility(4, 3, False, 2)


PINS = [
    pin_rms_norm_library, pin_rms_norm_closed_form, pin_rope_complex_form, pin_rope_hand_case,
    pin_rope_invariants, pin_qk_norm_then_rope, pin_projection_library, pin_context_kv_structure,
    pin_attention_brute_force, pin_attention_library, pin_attention_closed_forms,
    pin_attention_permutations, pin_requests_independent, pin_visibility,
]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(_ns())


# ----------------------------------------------------------------------------- planted mistakes

def _mut_rms_no_eps(x, w, eps):
    return O.rms_norm(x, w, 0.0)


def _mut_rms_gemma(x, w, eps):
    return O.rms_norm(x, 1.0 + np.asarray(w), eps)


def _mut_rms_sum(x, w, eps):
    return O.rms_norm(x, w, eps) / math.sqrt(np.asarray(x).shape[-1])


def _mut_rope_sign(x, pos, theta):
    return O.rope_neox(x, -np.asarray(pos), theta)


def _mut_rope_interleaved(x, pos, theta):
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])
    inv = np.argsort(perm)
    return O.rope_neox(x[..., perm], pos, theta)[..., inv]


def _mut_rope_freq(x, pos, theta):
    return O.rope_neox(x, pos, theta ** 0.5)


def _mut_qk_order(q, k, wq, wk, pos, eps, theta):
    kh = O.rms_norm(O.rope_neox(k, pos, theta), wk, eps)
    if q is None:
        return None, kh
    return O.rms_norm(O.rope_neox(q, pos, theta), wq, eps), kh


def _mut_attn_gqa_mod(q, kb, vb, kc, vc, cu_c, cu_b, scale, causal=False, window=0):
    # q-head h reads kv-head h % Hkv instead of h // (Hq/Hkv)
    q = np.asarray(q)
    hkv = np.shape(kb)[1]
    out = np.empty(q.shape)
    for h in range(q.shape[1]):
        g = h % hkv
        out[:, h:h + 1] = O.block_attention(q[:, h:h + 1], kb[:, g:g + 1], vb[:, g:g + 1],
                                            kc[:, g:g + 1], vc[:, g:g + 1], cu_c, cu_b, scale,
                                            causal, window)
    return out


def _mut_attn_swap_kv(q, kb, vb, kc, vc, cu_c, cu_b, scale, causal=False, window=0):
    return O.block_attention(q, vb, kb, vc, kc, cu_c, cu_b, scale, causal, window)


def _vis_off_by_one(ctx_len, blk_len, causal, window):
    n = ctx_len + blk_len
    vis = np.ones((blk_len, n), dtype=bool)
    if causal:
        qi = ctx_len + np.arange(blk_len).reshape(-1, 1)
        kj = np.arange(n).reshape(1, -1)
        vis = kj < qi + (qi == ctx_len)  # drops the diagonal except for the first row
        if window > 0:
            vis &= (qi - kj) <= window
    return vis


def _vis_window_inclusive(ctx_len, blk_len, causal, window):
    n = ctx_len + blk_len
    vis = np.ones((blk_len, n), dtype=bool)
    if causal:
        qi = ctx_len + np.arange(blk_len).reshape(-1, 1)
        kj = np.arange(n).reshape(1, -1)
        vis = kj <= qi
        if window > 0:
            vis &= (qi - kj) <= window
    return vis


def _mut_attn_no_scale(q, kb, vb, kc, vc, cu_c, cu_b, scale, causal=False, window=0):
    return O.block_attention(q, kb, vb, kc, vc, cu_c, cu_b, 1.0 if scale != 0 else 0.0, causal, window)


def _mut_proj_wk_for_v(h, wn, wk, wv, eps):
    k, _ = O.context_projection(h, wn, wk, wv, eps)
    return k, O.context_projection(h, wn, wk, wk, eps)[1]


def _mut_proj_no_hidden_norm(h, wn, wk, wv, eps):
    return O.context_projection(h, np.ones_like(np.asarray(wn)), wk, wv, eps)


MUTANTS = {
    "rms_no_eps": dict(rms_norm=_mut_rms_no_eps),
    "rms_gemma_weight": dict(rms_norm=_mut_rms_gemma),
    "rms_sum_not_mean": dict(rms_norm=_mut_rms_sum),
    "rope_sign": dict(rope_neox=_mut_rope_sign),
    "rope_interleaved_pairs": dict(rope_neox=_mut_rope_interleaved),
    "rope_wrong_freq": dict(rope_neox=_mut_rope_freq),
    "qk_rope_before_norm": dict(qk_norm_rope=_mut_qk_order),
    "attn_gqa_modulo": dict(block_attention=_mut_attn_gqa_mod),
    "attn_k_v_swapped": dict(block_attention=_mut_attn_swap_kv),
    "attn_no_scale": dict(block_attention=_mut_attn_no_scale),
    "proj_v_uses_wk": dict(context_projection=_mut_proj_wk_for_v),
    "proj_no_hidden_norm_weight": dict(context_projection=_mut_proj_no_hidden_norm),
}

INTERNAL_MUTANTS = {
    "mask_off_by_one": _vis_off_by_one,
    "window_inclusive": _vis_window_inclusive,
}


def _some_pin_fails(ns):
    for pin in PINS:
        try:
            pin(ns)
        except (AssertionError, ValueError):
            return pin.__name__
    return None


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(name):
    ns = _ns(**MUTANTS[name])
    # the composite functions route through the mutated pieces too
    if "rms_norm" in MUTANTS[name] or "rope_neox" in MUTANTS[name]:
        ns.qk_norm_rope = lambda q, k, wq, wk, pos, eps, th: _compose_qk(ns, q, k, wq, wk, pos, eps, th)
    if "context_projection" in MUTANTS[name]:
        ns.context_kv = lambda *a: _compose_ckv(ns, *a)
    assert _some_pin_fails(ns) is not None, f"no pin detects mutant {name}"


@pytest.mark.parametrize("name", sorted(INTERNAL_MUTANTS))
def test_pins_catch_planted_mask_mistakes(name, monkeypatch):
    monkeypatch.setattr(O, "attention_visibility", INTERNAL_MUTANTS[name])
    ns = _ns(attention_visibility=INTERNAL_MUTANTS[name])
    assert _some_pin_fails(ns) is not None, f"no pin detects mutant {name}"


def _compose_qk(ns, q, k, wq, wk, pos, eps, theta):
    kh = ns.rope_neox(ns.rms_norm(k, wk, eps), pos, theta)
    if q is None:
        return None, kh
    return ns.rope_neox(ns.rms_norm(q, wq, eps), pos, theta), kh


def _compose_ckv(ns, h, wn, wk, wv, wkn, pos, hkv, d, eps, theta):
    kr, v = ns.context_projection(h, wn, wk, wv, eps)
    c = kr.shape[0]
    _, kh = ns.qk_norm_rope(None, kr.reshape(c, hkv, d), None, wkn, pos, eps, theta)
    return kh, v.reshape(c, hkv, d)


def test_oracle_package_exports():
    for name in ("rms_norm", "rope_neox", "qk_norm_rope", "context_kv", "block_attention",
                 "draft_block_attention", "paged_context_rows"):
        assert callable(getattr(oracle, name))


# ---------------------------------------------------------------- paged context store

def _paged_fixture(seed=5, page=16):
    rng = np.random.default_rng(seed)
    ctx_lens = np.array([0, 1, 15, 16, 17, 40], dtype=np.int64)
    rows = rng.standard_normal((int(ctx_lens.sum()), 3, 4))
    npages = [(int(c) + page - 1) // page for c in ctx_lens]
    total = sum(npages) + 3
    perm = rng.permutation(total)
    bt = np.full((len(ctx_lens), max(npages)), -1, dtype=np.int64)
    nxt = 0
    slots = []
    for r, c in enumerate(ctx_lens.tolist()):
        for p_ in range(npages[r]):
            bt[r, p_] = perm[nxt]
            nxt += 1
        slots += [bt[r, k // page] * page + k % page for k in range(c)]
    pool = np.full((total * page, 3, 4), np.nan)
    pool[np.array(slots, dtype=np.int64)] = rows       # flat-slot scatter, written independently
    return pool.reshape(total, page, 3, 4), bt, ctx_lens, rows


def test_paged_rows_round_trip():
    # rows scattered to flat slots (page * 16 + offset) come back in order
    pool, bt, lens, rows = _paged_fixture()
    got = O.paged_context_rows(pool, bt, lens)
    assert got.shape == rows.shape and np.array_equal(got, rows)


def test_paged_rows_identity_table():
    # the pages' own store: one request, identity table, row p at flat slot p
    rng = np.random.default_rng(9)
    flat = rng.standard_normal((5 * 16, 2, 3))
    got = O.paged_context_rows(flat.reshape(5, 16, 2, 3), np.arange(5)[None, :], [70])
    assert np.array_equal(got, flat[:70])


def test_paged_rows_pin_catches_index_mistakes():
    pool, bt, lens, rows = _paged_fixture()

    def wrong_offset(pool, bt, lens, page=16):  # offset taken from the wrong end of the page
        return np.stack([pool[int(bt[r][k // page]), page - 1 - k % page]
                         for r, c in enumerate(lens) for k in range(int(c))])

    def wrong_page(pool, bt, lens, page=16):  # pages counted from 1
        return np.stack([pool[int(bt[r][min(k // page + 1, bt.shape[1] - 1)]), k % page]
                         for r, c in enumerate(lens) for k in range(int(c))])

    for f in (wrong_offset, wrong_page):
        got = f(pool, bt, lens)
        assert not np.array_equal(got, rows)


# ---------------------------------------------------------------- the layer around the attention

def _layer_ns(**over):
    base = dict(residual_rms_norm=O.residual_rms_norm, block_qkv=O.block_qkv,
                output_projection=O.output_projection)
    base.update(over)
    return types.SimpleNamespace(**base)


def lpin_residual_norm(X):
    t, h = 6, 40
    x = RNG.standard_normal((t, h))
    r = RNG.standard_normal((t, h))
    w = RNG.uniform(0.5, 1.5, h)
    res, normed = X.residual_rms_norm(x, r, w, 1e-6)
    assert np.array_equal(res, x + r)                   # the residual stream becomes the sum
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x + r), (h,), torch.from_numpy(w), eps=1e-6)
    np.testing.assert_allclose(normed, ref.numpy(), rtol=1e-13, atol=1e-13)
    res0, normed0 = X.residual_rms_norm(x, None, w, 1e-6)   # no residual: the norm of hidden
    assert np.array_equal(res0, x)
    ref0 = torch.nn.functional.rms_norm(torch.from_numpy(x), (h,), torch.from_numpy(w), eps=1e-6)
    np.testing.assert_allclose(normed0, ref0.numpy(), rtol=1e-13, atol=1e-13)


def lpin_block_qkv_split(X):
    # the merged weight's row blocks, each applied by the library's linear
    t, h, hq, hkv, d = 5, 24, 4, 2, 6
    x = RNG.standard_normal((t, h))
    wq = RNG.standard_normal((hq * d, h))
    wk = RNG.standard_normal((hkv * d, h))
    wv = RNG.standard_normal((hkv * d, h))
    q, k, v = X.block_qkv(x, np.concatenate([wq, wk, wv]), hq, hkv, d)
    lin = lambda w: torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(w)).numpy()
    np.testing.assert_allclose(q, lin(wq).reshape(t, hq, d), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(k, lin(wk).reshape(t, hkv, d), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(v, lin(wv).reshape(t, hkv, d), rtol=1e-12, atol=1e-12)
    # head h of q is rows [h Dh, (h + 1) Dh) of the weight: a weight that is
    # zero except one row of head 2 moves one input column to q[:, 2, e]
    w = np.zeros(((hq + 2 * hkv) * d, h))
    w[2 * d + 3, 7] = 1.0
    q1, k1, v1 = X.block_qkv(x, w, hq, hkv, d)
    assert np.array_equal(q1[:, 2, 3], x[:, 7]) and np.count_nonzero(q1) == np.count_nonzero(x[:, 7])
    assert not k1.any() and not v1.any()


def lpin_output_projection(X):
    t, hq, d, hsz = 4, 3, 5, 7
    a = RNG.standard_normal((t, hq, d))
    w = RNG.standard_normal((hsz, hq * d))
    ref = torch.nn.functional.linear(torch.from_numpy(a.reshape(t, hq * d)), torch.from_numpy(w))
    np.testing.assert_allclose(X.output_projection(a, w), ref.numpy(), rtol=1e-12, atol=1e-12)
    # head-major flattening: input column h * Dh + e is head h, element e
    w1 = np.zeros((hsz, hq * d))
    w1[0, 2 * d + 1] = 1.0
    np.testing.assert_array_equal(X.output_projection(a, w1)[:, 0], a[:, 2, 1])


def lpin_layer_reduces_to_attention(X):
    # H = Hq Dh, q weight = identity, o_proj = identity, unit norm weight:
    # the layer is the block attention of the normed rows with k = x Wk^T, v = x Wv^T
    hq, hkv, d = 2, 1, 8
    h = hq * d
    cu_c = np.array([0, 5, 12])
    cu_b = np.array([0, 3, 7])
    t = int(cu_b[-1])
    x = RNG.standard_normal((t, h))
    wk = RNG.standard_normal((hkv * d, h)) * 0.3
    wv = RNG.standard_normal((hkv * d, h)) * 0.3
    w_qkv = np.concatenate([np.eye(h), wk, wv])
    kc = RNG.standard_normal((int(cu_c[-1]), hkv, d))
    vc = RNG.standard_normal((int(cu_c[-1]), hkv, d))
    pos = np.concatenate([np.arange(c, c + b) for c, b in zip(np.diff(cu_c), np.diff(cu_b))])
    ones = np.ones(d)
    o, res, q, k, v, attn = O.draft_layer_attention(
        x, None, np.ones(h), w_qkv, np.eye(h), pos, kc, vc, cu_c, cu_b, ones, ones, hq, hkv, d,
        1e-6, 1e4, d ** -0.5)
    _, normed = X.residual_rms_norm(x, None, np.ones(h), 1e-6)
    ref, _, _ = O.draft_block_attention(normed.reshape(t, hq, d), (normed @ wk.T).reshape(t, hkv, d),
                                        (normed @ wv.T).reshape(t, hkv, d), pos, kc, vc, cu_c, cu_b,
                                        ones, ones, 1e-6, 1e4, d ** -0.5)
    np.testing.assert_allclose(o, ref.reshape(t, h), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(attn, ref, rtol=1e-12, atol=1e-12)


LAYER_PINS = [lpin_residual_norm, lpin_block_qkv_split, lpin_output_projection,
              lpin_layer_reduces_to_attention]


@pytest.mark.parametrize("pin", LAYER_PINS, ids=[p.__name__ for p in LAYER_PINS])
def test_layer_oracle_pin(pin):
    pin(_layer_ns())


def _lmut_no_residual(x, r, w, eps):
    return O.residual_rms_norm(x, None, w, eps)


def _lmut_norm_before_add(x, r, w, eps):
    res, normed = O.residual_rms_norm(x, None, w, eps)
    return (res if r is None else res + r), normed


def _lmut_kv_swapped(x, w, hq, hkv, d):
    q, k, v = O.block_qkv(x, w, hq, hkv, d)
    return q, v, k


def _lmut_heads_transposed(x, w, hq, hkv, d):
    q, k, v = O.block_qkv(x, w, hq, hkv, d)
    t = q.shape[0]
    return q.reshape(t, d, hq).transpose(0, 2, 1), k, v


def _lmut_oproj_dim_major(a, w):
    a = np.asarray(a, np.float64)
    return a.transpose(0, 2, 1).reshape(a.shape[0], -1) @ np.asarray(w, np.float64).T


def _lmut_oproj_no_transpose(a, w):
    a = np.asarray(a, np.float64)
    w = np.asarray(w, np.float64)
    return a.reshape(a.shape[0], -1) @ w.reshape(w.shape[1], w.shape[0])


LAYER_MUTANTS = {
    "residual_dropped": dict(residual_rms_norm=_lmut_no_residual),
    "norm_before_residual_add": dict(residual_rms_norm=_lmut_norm_before_add),
    "qkv_k_v_swapped": dict(block_qkv=_lmut_kv_swapped),
    "qkv_heads_transposed": dict(block_qkv=_lmut_heads_transposed),
    "oproj_dim_major_flatten": dict(output_projection=_lmut_oproj_dim_major),
    "oproj_weight_not_transposed": dict(output_projection=_lmut_oproj_no_transpose),
}


@pytest.mark.parametrize("name", sorted(LAYER_MUTANTS))
def test_layer_pins_catch_planted_mistakes(name):
    ns = _layer_ns(**LAYER_MUTANTS[name])
    failed = False
    for pin in LAYER_PINS:
        try:
            pin(ns)
        except (AssertionError, ValueError):
            failed = True
            break
    assert failed, f"no layer pin detects mutant {name}"


# ---------------------------------------------------------------- propose-step preparation

def _prep_example(sample_from_anchor=False, max_model_len=100, prep=None):
    prep = prep or O.prepare_dflash_inputs
    nqpr = 3
    return prep(
        idx_mapping=[1, 0], target_query_start_loc=[0, 3, 4], target_positions=[5, 6, 7, 0],
        num_rejected=[1, 0], num_sampled=[1, 0], last_sampled=[11, 42], next_prefill_tokens=[17, 99],
        block_table=[[9, 3, 7], [2, 5, 6]], num_query_per_req=nqpr,
        num_speculative_steps=nqpr if sample_from_anchor else nqpr - 1, block_size=4,
        max_num_reqs=3, max_num_tokens=8, max_model_len=max_model_len, mask_token_id=-5,
        sample_from_anchor=sample_from_anchor)


def ppin_hand_example(prep):
    # worked by hand: request 0 (state 1) keeps positions 5, 6 of its three
    # verified rows (one rejected), sampled before -> anchor last_sampled[1] = 42
    # at position 7; request 1 (state 0) has one prefill row at position 0 and
    # sampled nothing -> anchor next_prefill_tokens[0] = 17 at position 1.
    o = _prep_example(prep=prep)
    eq = lambda k, v: np.testing.assert_array_equal(o[k], np.array(v), err_msg=k)
    eq("context_positions", [5, 6, 7, 0])
    eq("context_slot_mapping", [3 * 4 + 1, 3 * 4 + 2, 3 * 4 + 3, 2 * 4 + 0])
    eq("input_ids", [42, -5, -5, 17, -5, -5])
    eq("query_positions", [7, 8, 9, 1, 2, 3])
    eq("query_slot_mapping", [3 * 4 + 3, 7 * 4 + 0, 7 * 4 + 1, 2 * 4 + 1, 2 * 4 + 2, 2 * 4 + 3, -1, -1])
    eq("query_start_loc", [0, 3, 6, 6])
    eq("seq_lens", [6 + 1 + 3, 0 + 1 + 3, 0])
    eq("sample_indices", [1, 2, 4, 5, 0, 0])
    eq("sample_pos", [8, 9, 2, 3, 0, 0])
    eq("sample_idx_mapping", [1, 1, 0, 0, -1, -1])
    eq("ctx_cu", [0, 7, 8, 8])                         # kept context rows: 0..6 and 0


def ppin_sample_from_anchor_and_clamps(prep):
    o = _prep_example(sample_from_anchor=True, max_model_len=9, prep=prep)
    np.testing.assert_array_equal(o["query_positions"], [7, 8, 8, 1, 2, 3])     # min(pos, 8)
    np.testing.assert_array_equal(o["sample_indices"], [0, 1, 2, 3, 4, 5, 0, 0, 0])
    np.testing.assert_array_equal(o["sample_pos"], [8, 9, 10, 2, 3, 4, 0, 0, 0])
    np.testing.assert_array_equal(o["sample_idx_mapping"], [1, 1, 1, 0, 0, 0, -1, -1, -1])
    # positions past the table's last page use the last page
    o2 = prep(idx_mapping=[0], target_query_start_loc=[0, 1], target_positions=[14],
              num_rejected=[0], num_sampled=[1], last_sampled=[3], next_prefill_tokens=[0],
              block_table=[[4, 8]], num_query_per_req=2, num_speculative_steps=1, block_size=4,
              max_num_reqs=1, max_num_tokens=2, max_model_len=100, mask_token_id=0,
              sample_from_anchor=False)
    np.testing.assert_array_equal(o2["context_slot_mapping"], [8 * 4 + 2])
    np.testing.assert_array_equal(o2["query_slot_mapping"], [8 * 4 + 3, 8 * 4 + 0])


PREP_PINS = [ppin_hand_example, ppin_sample_from_anchor_and_clamps]


@pytest.mark.parametrize("pin", PREP_PINS, ids=[p.__name__ for p in PREP_PINS])
def test_prep_oracle_pin(pin):
    pin(O.prepare_dflash_inputs)


def _prep_mutant(**change):
    def f(**kw):
        if change.get("no_rollback"):
            kw = dict(kw, num_rejected=[0] * len(kw["num_rejected"]))
        if change.get("anchor_always_last"):
            kw = dict(kw, num_sampled=[1] * len(kw["num_sampled"]))
        o = O.prepare_dflash_inputs(**kw)
        if change.get("no_position_clamp"):
            o["query_positions"] = O.prepare_dflash_inputs(**dict(kw, max_model_len=1 << 40))["query_positions"]
        if change.get("sample_pos_shift"):
            o["sample_pos"] = o["sample_pos"] + (o["sample_idx_mapping"] >= 0)
        return o
    return f


PREP_MUTANTS = {
    "no_rollback": dict(no_rollback=True),
    "anchor_always_last_sampled": dict(anchor_always_last=True),
    "no_position_clamp": dict(no_position_clamp=True),
    "sample_pos_off_by_one": dict(sample_pos_shift=True),
}


@pytest.mark.parametrize("name", sorted(PREP_MUTANTS))
def test_prep_pins_catch_planted_mistakes(name):
    f = _prep_mutant(**PREP_MUTANTS[name])
    failed = False
    for pin in PREP_PINS:
        try:
            pin(f)
        except AssertionError:
            failed = True
            break
    assert failed, f"no prep pin detects mutant {name}"


def test_fc_combine_and_bf16_round_pins():
    # bf16 rounding against the library's cast; fc against the library's linear
    x = RNG.standard_normal(1000).astype(np.float32) * np.float32(7.3)
    x[:4] = [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -0.0, 3.0e38]   # ties to even, sign, large
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.bf16_round(x), ref)
    t, h, taps = 5, 8, 3
    aux = RNG.standard_normal((t, h * taps))
    w = RNG.standard_normal((h, h * taps))
    np.testing.assert_allclose(O.fc_combine(aux, w),
                               torch.nn.functional.linear(torch.from_numpy(aux), torch.from_numpy(w)).numpy(),
                               rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- composed functions
# draft_block_attention and draft_layer_attention are the reference of every
# GPU attention parity test. They are pinned here with distinct, non-unit q,
# k and input-norm weights and non-trivial positions against a composition of
# independent pieces: torch's fp64 rms_norm and linear, RoPE in its complex
# form (x_i + i x_{i+Dh/2}) e^{i p theta^(-2i/Dh)}, and torch's
# scaled_dot_product_attention with an explicit mask over [context; block].

def _ref_rope_complex(x, pos, theta):
    x = np.asarray(x, np.float64)
    half = x.shape[-1] // 2
    inv = float(theta) ** (-2.0 * np.arange(half) / x.shape[-1])
    z = (x[..., :half] + 1j * x[..., half:]) * np.exp(1j * np.outer(pos, inv))[:, None, :]
    return np.concatenate([z.real, z.imag], axis=-1)


def _ref_head_norm(x, w, eps):
    t = torch.from_numpy(np.asarray(x, np.float64))
    return torch.nn.functional.rms_norm(t, (t.shape[-1],), torch.from_numpy(np.asarray(w, np.float64)),
                                        eps=eps).numpy()


def _ref_sdpa(qh, kh, vb, kc, vc, cu_c, cu_b, scale, causal, window):
    out = np.zeros_like(qh)
    for r in range(len(cu_b) - 1):
        c0, c1, b0, b1 = int(cu_c[r]), int(cu_c[r + 1]), int(cu_b[r]), int(cu_b[r + 1])
        n, bl = c1 - c0 + b1 - b0, b1 - b0
        keys = torch.from_numpy(np.concatenate([kc[c0:c1], kh[b0:b1]])).permute(1, 0, 2).contiguous()
        vals = torch.from_numpy(np.concatenate([vc[c0:c1], vb[b0:b1]])).permute(1, 0, 2).contiguous()
        qq = torch.from_numpy(qh[b0:b1]).permute(1, 0, 2).contiguous()
        qi = torch.arange(bl).reshape(-1, 1) + (c1 - c0)
        kj = torch.arange(n).reshape(1, -1)
        mask = torch.ones(bl, n, dtype=torch.bool)
        if causal:
            mask = kj <= qi
            if window > 0:
                mask &= (qi - kj) < window
        o = torch.nn.functional.scaled_dot_product_attention(qq, keys, vals, attn_mask=mask,
                                                             scale=scale, enable_gqa=True)
        out[b0:b1] = o.permute(1, 0, 2).numpy()
    return out


def _comp_batch(seed):
    rng = np.random.default_rng(seed)
    hq, hkv, d = 6, 2, 8
    cu_c, cu_b = np.array([0, 11, 11, 30]), np.array([0, 4, 9, 12])
    t, c = int(cu_b[-1]), int(cu_c[-1])
    # block positions not at the context's end, one request's reversed
    pos = np.concatenate([np.arange(int(cu_c[r + 1] - cu_c[r]), int(cu_c[r + 1] - cu_c[r] + cu_b[r + 1] - cu_b[r]))
                          + 5 * r for r in range(3)])
    pos[4:9] = pos[4:9][::-1]
    return dict(
        hq=hq, hkv=hkv, d=d, cu_c=cu_c, cu_b=cu_b, pos=pos,
        q=rng.standard_normal((t, hq, d)) * 2.0, kb=rng.standard_normal((t, hkv, d)) * 0.5,
        vb=rng.standard_normal((t, hkv, d)), kc=rng.standard_normal((c, hkv, d)),
        vc=rng.standard_normal((c, hkv, d)),
        wq=rng.uniform(0.5, 1.5, d), wk=rng.uniform(0.5, 1.5, d) + 0.75,
        theta=500.0, eps=1e-6, scale=0.41, rng=rng)


def _comp_ns(**over):
    base = dict(draft_block_attention=O.draft_block_attention,
                draft_layer_attention=O.draft_layer_attention)
    base.update(over)
    return types.SimpleNamespace(**base)


def cpin_draft_block_attention(X):
    b = _comp_batch(77)
    for causal, window in ((False, 0), (True, 0), (True, 6)):
        out, qh, kh = X.draft_block_attention(b["q"], b["kb"], b["vb"], b["pos"], b["kc"], b["vc"],
                                              b["cu_c"], b["cu_b"], b["wq"], b["wk"], b["eps"],
                                              b["theta"], b["scale"], causal, window)
        rq = _ref_rope_complex(_ref_head_norm(b["q"], b["wq"], b["eps"]), b["pos"], b["theta"])
        rk = _ref_rope_complex(_ref_head_norm(b["kb"], b["wk"], b["eps"]), b["pos"], b["theta"])
        np.testing.assert_allclose(qh, rq, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(kh, rk, rtol=1e-12, atol=1e-12)
        ref = _ref_sdpa(rq, rk, b["vb"], b["kc"], b["vc"], b["cu_c"], b["cu_b"], b["scale"],
                        causal, window)
        np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)


def cpin_draft_layer_attention(X):
    b = _comp_batch(78)
    rng = b["rng"]
    hq, hkv, d = b["hq"], b["hkv"], b["d"]
    h, t = 20, int(b["cu_b"][-1])
    x, res_in = rng.standard_normal((t, h)), rng.standard_normal((t, h))
    w_in = rng.uniform(0.5, 1.5, h)
    w_qkv = rng.standard_normal(((hq + 2 * hkv) * d, h)) * 0.4
    w_o = rng.standard_normal((h, hq * d)) * 0.3
    for causal, window in ((False, 0), (True, 5)):
        o, res, q, k, v, attn = X.draft_layer_attention(
            x, res_in, w_in, w_qkv, w_o, b["pos"], b["kc"], b["vc"], b["cu_c"], b["cu_b"], b["wq"],
            b["wk"], hq, hkv, d, b["eps"], b["theta"], b["scale"], causal, window)
        tt = lambda a: torch.from_numpy(np.asarray(a, np.float64))
        r_res = x + res_in
        normed = torch.nn.functional.rms_norm(tt(r_res), (h,), tt(w_in), eps=b["eps"])
        qkv = torch.nn.functional.linear(normed, tt(w_qkv)).numpy()
        rq = qkv[:, :hq * d].reshape(t, hq, d)
        rk = qkv[:, hq * d:(hq + hkv) * d].reshape(t, hkv, d)
        rv = qkv[:, (hq + hkv) * d:].reshape(t, hkv, d)
        qh = _ref_rope_complex(_ref_head_norm(rq, b["wq"], b["eps"]), b["pos"], b["theta"])
        kh = _ref_rope_complex(_ref_head_norm(rk, b["wk"], b["eps"]), b["pos"], b["theta"])
        ra = _ref_sdpa(qh, kh, rv, b["kc"], b["vc"], b["cu_c"], b["cu_b"], b["scale"], causal, window)
        ro = torch.nn.functional.linear(tt(ra.reshape(t, hq * d)), tt(w_o)).numpy()
        np.testing.assert_array_equal(res, r_res)
        for got, ref in ((q, rq), (k, rk), (v, rv)):
            np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(attn, ra, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(o, ro, rtol=1e-11, atol=1e-12)


COMPOSED_PINS = [cpin_draft_block_attention, cpin_draft_layer_attention]


@pytest.mark.parametrize("pin", COMPOSED_PINS, ids=[p.__name__ for p in COMPOSED_PINS])
def test_composed_oracle_pin(pin):
    pin(_comp_ns())


def _cmut_block_qk_weights_swapped(q, kb, vb, pos, kc, vc, cu_c, cu_b, wq, wk, *rest):
    return O.draft_block_attention(q, kb, vb, pos, kc, vc, cu_c, cu_b, wk, wq, *rest)


def _cmut_block_no_rope(q, kb, vb, pos, kc, vc, cu_c, cu_b, *rest):
    return O.draft_block_attention(q, kb, vb, np.zeros_like(pos), kc, vc, cu_c, cu_b, *rest)


def _cmut_block_q_weight_for_both(q, kb, vb, pos, kc, vc, cu_c, cu_b, wq, wk, *rest):
    return O.draft_block_attention(q, kb, vb, pos, kc, vc, cu_c, cu_b, wq, wq, *rest)


def _cmut_layer_qk_weights_swapped(x, r, w_in, w_qkv, w_o, pos, kc, vc, cu_c, cu_b, wq, wk, *rest):
    return O.draft_layer_attention(x, r, w_in, w_qkv, w_o, pos, kc, vc, cu_c, cu_b, wk, wq, *rest)


def _cmut_layer_unit_input_norm(x, r, w_in, *rest):
    return O.draft_layer_attention(x, r, np.ones_like(w_in), *rest)


def _cmut_layer_no_residual(x, r, *rest):
    return O.draft_layer_attention(x, None, *rest)


COMPOSED_MUTANTS = {
    "block_q_k_norm_weights_swapped": dict(draft_block_attention=_cmut_block_qk_weights_swapped),
    "block_rope_at_position_zero": dict(draft_block_attention=_cmut_block_no_rope),
    "block_q_norm_weight_on_k": dict(draft_block_attention=_cmut_block_q_weight_for_both),
    "layer_q_k_norm_weights_swapped": dict(draft_layer_attention=_cmut_layer_qk_weights_swapped),
    "layer_input_norm_weight_dropped": dict(draft_layer_attention=_cmut_layer_unit_input_norm),
    "layer_residual_dropped": dict(draft_layer_attention=_cmut_layer_no_residual),
}


@pytest.mark.parametrize("name", sorted(COMPOSED_MUTANTS))
def test_composed_pins_catch_planted_mistakes(name):
    ns = _comp_ns(**COMPOSED_MUTANTS[name])
    failed = []
    for pin in COMPOSED_PINS:
        try:
            pin(ns)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no composed pin detects mutant {name}"
