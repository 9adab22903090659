"""Randomised pins of the fp64 oracle (CPU only).

hypothesis draws small batch shapes (empty contexts and blocks included), head
geometries, masks, scales, positions and RoPE bases, and the oracle's block
attention, its q/k norm + RoPE and its context K/V projection must agree with
the independent formulations the fixed pins use: the explicit-loop brute force
and torch's scaled_dot_product_attention with an explicit mask for the
attention, RoPE in complex form over torch's rms_norm for the rotation, torch's
rms_norm and linear for the projection. The draws are derandomised, so every
run checks the same examples.
"""
import numpy as np
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle import dflash_oracle as O
from test_oracle_pins import _brute, _rand_batch, _ref_head_norm, _ref_rope_complex, _ref_sdpa

SET = settings(max_examples=60, deadline=None, derandomize=True,
               suppress_health_check=list(HealthCheck))


@st.composite
def _batches(draw):
    r = draw(st.integers(1, 3))
    ctx = draw(st.lists(st.integers(0, 12), min_size=r, max_size=r))
    blk = draw(st.lists(st.integers(0, 6), min_size=r, max_size=r))
    hkv = draw(st.integers(1, 3))
    group = draw(st.integers(1, 3))
    d = draw(st.sampled_from([2, 4, 8]))
    causal = draw(st.booleans())
    window = draw(st.integers(0, 8)) if causal else 0
    scale = draw(st.floats(0.05, 1.5))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    return ctx, blk, hkv * group, hkv, d, causal, window, scale, seed


@SET
@given(_batches())
def test_block_attention_matches_brute_force_and_sdpa(b):
    ctx, blk, hq, hkv, d, causal, window, scale, seed = b
    args = _rand_batch(ctx, blk, hq, hkv, d, seed)
    got = O.block_attention(*args, scale, causal, window)
    np.testing.assert_allclose(got, _brute(*args, scale, causal, window), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(got, _ref_sdpa(*args, scale, causal, window), rtol=1e-10, atol=1e-11)


@SET
@given(st.integers(1, 20), st.integers(0, 6), st.integers(1, 4), st.sampled_from([2, 4, 8, 16]),
       st.integers(0, 2 ** 31 - 1), st.sampled_from([1e4, 1e6]))
def test_qk_norm_rope_matches_the_complex_form(t, hq, hkv, d, seed, theta):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((t, hq, d)) if hq else None
    k = rng.standard_normal((t, hkv, d))
    wq, wk = rng.uniform(0.5, 1.5, d), rng.uniform(0.5, 1.5, d)
    pos = rng.integers(0, 40000, t)
    qo, ko = O.qk_norm_rope(q, k, wq if hq else None, wk, pos, 1e-6, theta)
    np.testing.assert_allclose(ko, _ref_rope_complex(_ref_head_norm(k, wk, 1e-6), pos, theta),
                               rtol=1e-9, atol=1e-10)
    if hq:
        np.testing.assert_allclose(qo, _ref_rope_complex(_ref_head_norm(q, wq, 1e-6), pos, theta),
                                   rtol=1e-9, atol=1e-10)
    else:
        assert qo is None


@SET
@given(st.integers(1, 12), st.sampled_from([4, 8, 16, 32]), st.integers(1, 3), st.sampled_from([2, 4, 8]),
       st.integers(0, 2 ** 31 - 1))
def test_context_kv_matches_a_composition(rows, hidden, hkv, d, seed):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((rows, hidden))
    wn, wkn = rng.uniform(0.5, 1.5, hidden), rng.uniform(0.5, 1.5, d)
    wk, wv = rng.standard_normal((hkv * d, hidden)) * 0.1, rng.standard_normal((hkv * d, hidden)) * 0.1
    pos = rng.integers(0, 5000, rows)
    k, v = O.context_kv(h, wn, wk, wv, wkn, pos, hkv, d, 1e-6, 1e6)
    n = torch.nn.functional.rms_norm(torch.from_numpy(h), (hidden,), torch.from_numpy(wn), eps=1e-6)
    kr = torch.nn.functional.linear(n, torch.from_numpy(wk)).numpy().reshape(rows, hkv, d)
    vr = torch.nn.functional.linear(n, torch.from_numpy(wv)).numpy().reshape(rows, hkv, d)
    np.testing.assert_allclose(v, vr, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(k, _ref_rope_complex(_ref_head_norm(kr, wkn, 1e-6), pos, 1e6),
                               rtol=1e-9, atol=1e-10)
