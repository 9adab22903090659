"""Plain, slow, fp64 CPU oracle of the DFlash draft block-attention path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path. It
shares no code, header, table or helper with the HIP library.

Everything is computed in float64 from the exact input values (bf16 or f32
inputs are widened without change). There is no intermediate rounding, no
blocking, no fusion and no online softmax: each function is the plain
definition of its step, written in the order the pages apply the steps.

Sources (pages of the vllm.cpp project):
  * "qwen3_dflash.cpp" page -- file header (the block attention is the one new
    operation; full-attention layers are bidirectional inside the block, sliding
    window layers causal with a window), ``PrecomputeContextKVDevice`` (hidden
    RMSNorm, K/V projection as rows of the merged qkv weight, per-head k-norm,
    NeoX RoPE at context positions, V raw), ``ForwardBlockLogits`` and
    ``ForwardWithCtxKVDev`` (per-head q/k RMSNorm, NeoX RoPE at block positions,
    scale 1/sqrt(Dh), attention of each block over its request's
    [context; block] sequence, only block-query rows kept).
  * "qwen3.cpp" page -- file header (standard, non-gemma RMSNorm; q/k norm
    applied before RoPE).
  * "qwen3_dflash.cpp" page, the paged draft-KV store read by
    ``ForwardPagedBody``: pools of fixed-size pages, a per-request block table
    of page ids; context row p of a request lives at page p // page_size,
    offset p % page_size.
  * "qwen3_dflash.cpp" page, ``PrepareDflashInputs`` (integer preparation of
    a propose step: context rows and their slots, rollback of rejected
    drafts, the anchor + mask block, sample maps, padding) and
    ``CombineAuxFeatures`` (the multi-tap fc combine).
  * "qwen3_dflash.cpp" page, ``ForwardBlockLogits`` and ``ForwardWithCtxKVDev``
    (the layer around the attention): input_layernorm as the standard
    residual add + RMSNorm, the merged qkv weight applied as one product and
    split into q | k | v, and o_proj applied to the attention output.

Readings taken where the pages are silent:
  * GQA: q-head h reads kv-head h // (Hq/Hkv).
  * NeoX RoPE pairs element i with element i + Dh/2; inverse frequency
    theta**(-2i/Dh); the whole head dimension rotates.
  * The mask is defined on the index in the per-request combined sequence
    [context rows 0..C-1; block rows C..C+B-1], the only thing the pages hand the
    attention (cumulative sequence lengths). Bidirectional: every key visible.
    Causal: key k visible to query i iff k <= i; with a window W > 0 also
    i - k < W (W keys including the query's own row).
  * A query row with no visible key yields 0 (cannot happen when B >= 1).

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``
against closed forms, invariants, library routines and brute force. No
function is "parity unpinned" at the level of its definition; the pairing
convention of RoPE is fixed only by the name "NeoX" on the pages (both
pairings satisfy the invariants the pins check).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "rms_norm",
    "rope_inv_freq",
    "rope_neox",
    "qk_norm_rope",
    "context_projection",
    "context_kv",
    "attention_visibility",
    "block_attention",
    "draft_block_attention",
    "paged_context_rows",
    "residual_rms_norm",
    "block_qkv",
    "output_projection",
    "draft_layer_attention",
    "PAD_SLOT",
    "prepare_dflash_inputs",
    "fc_combine",
    "bf16_round",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def rms_norm(x, w, eps):
    """Standard RMSNorm over the last axis: ``x * w / sqrt(mean(x**2) + eps)``.

    "qwen3_dflash.cpp" page, ``PrecomputeContextKVDevice`` (hidden_norm and
    k_norm) and ``ForwardBlockLogits`` (q_norm, k_norm over head_dim), both
    with the non-gemma flag; "qwen3.cpp" page header (standard RMSNorm, weight
    multiplies directly, no 1 + w).
    """
    x = _f64(x)
    w = _f64(w)
    mean_sq = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(mean_sq + float(eps)) * w


def rope_inv_freq(head_dim, theta):
    """Inverse frequencies ``theta ** (-2 i / Dh)`` for i in [0, Dh/2)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return float(theta) ** (-(2.0 * i) / float(head_dim))


def rope_neox(x, positions, theta):
    """NeoX (rotate-half) rotary embedding.

    ``x`` is ``[T, H, Dh]``; ``positions`` is ``[T]`` integer. For each row t
    and pair index i < Dh/2, with angle a = positions[t] * inv_freq[i]:
    ``y[i] = x[i] cos a - x[i + Dh/2] sin a`` and
    ``y[i + Dh/2] = x[i + Dh/2] cos a + x[i] sin a``.

    "qwen3_dflash.cpp" page: ``RopeNeox`` applied to q and k at the block
    positions (``ForwardBlockLogits``) and to K at the context positions
    (``PrecomputeContextKVDevice``).
    """
    x = _f64(x)
    t, h, d = x.shape
    half = d // 2
    ang = _f64(positions).reshape(t, 1) * rope_inv_freq(d, theta).reshape(1, half)
    cos = np.cos(ang)[:, None, :]
    sin = np.sin(ang)[:, None, :]
    x1 = x[:, :, :half]
    x2 = x[:, :, half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def qk_norm_rope(q, k, q_norm_w, k_norm_w, positions, eps, theta):
    """Per-head RMSNorm of q and k over head_dim, then NeoX RoPE on both.

    ``q`` ``[T, Hq, Dh]`` (or None for the K-only form used on context rows),
    ``k`` ``[T, Hkv, Dh]``. Returns ``(q_hat or None, k_hat)``.

    "qwen3_dflash.cpp" page, ``ForwardBlockLogits``: q_norm then k_norm then
    RopeNeox(q, k, positions); "qwen3.cpp" page header: norm before RoPE.
    """
    k_hat = rope_neox(rms_norm(k, k_norm_w, eps), positions, theta)
    if q is None:
        return None, k_hat
    q_hat = rope_neox(rms_norm(q, q_norm_w, eps), positions, theta)
    return q_hat, k_hat


def context_projection(hidden, hidden_norm_w, w_k, w_v, eps):
    """Hidden RMSNorm then the K and V projections of the context rows.

    ``normed = RMSNorm(hidden, hidden_norm_w)``; ``K = normed @ w_k.T`` and
    ``V = normed @ w_v.T`` where ``w_k``/``w_v`` are ``[Hkv*Dh, H]`` (rows of
    the merged qkv weight). Returns ``(K_raw [C, Hkv*Dh], V [C, Hkv*Dh])``.

    "qwen3_dflash.cpp" page, ``PrecomputeContextKVDevice``: RmsNorm with
    hidden_norm, then MatmulBT against the K and V row slices.
    """
    normed = rms_norm(hidden, hidden_norm_w, eps)
    k_raw = normed @ _f64(w_k).T
    v = normed @ _f64(w_v).T
    return k_raw, v


def context_kv(hidden, hidden_norm_w, w_k, w_v, k_norm_w, positions,
               num_kv_heads, head_dim, eps, theta):
    """Context K/V precompute: projection, per-head k-norm, NeoX RoPE on K.

    Returns ``(K_hat [C, Hkv, Dh], V [C, Hkv, Dh])``; V is left raw.

    "qwen3_dflash.cpp" page, ``PrecomputeContextKVDevice`` and the
    ``ContextKVDev`` record (K normed and rotated, V raw).
    """
    k_raw, v = context_projection(hidden, hidden_norm_w, w_k, w_v, eps)
    c = k_raw.shape[0]
    k3 = k_raw.reshape(c, num_kv_heads, head_dim)
    _, k_hat = qk_norm_rope(None, k3, None, k_norm_w, positions, eps, theta)
    return k_hat, v.reshape(c, num_kv_heads, head_dim)


def attention_visibility(ctx_len, blk_len, causal, window):
    """Boolean ``[blk_len, ctx_len + blk_len]`` visibility of keys to block queries.

    Indices are positions in the per-request combined sequence: context rows
    0..ctx_len-1, then block rows ctx_len..ctx_len+blk_len-1. Block query b sits
    at index ctx_len + b. Bidirectional (``causal`` false): all keys visible.
    Causal: key k visible iff k <= query index; with ``window`` > 0 also
    ``query index - k < window``.

    "qwen3_dflash.cpp" page header: bidirectional in-block attention on full
    attention layers, causal plus sliding window on SWA layers; the attention
    receives only cumulative lengths, so the mask lives on these indices.
    """
    n = ctx_len + blk_len
    vis = np.ones((blk_len, n), dtype=bool)
    if causal:
        qi = ctx_len + np.arange(blk_len).reshape(-1, 1)
        kj = np.arange(n).reshape(1, -1)
        vis = kj <= qi
        if window > 0:
            vis &= (qi - kj) < window
    elif window > 0:
        raise ValueError("a sliding window is only defined for causal layers")
    return vis


def block_attention(q, k_blk, v_blk, k_ctx, v_ctx, cu_ctx, cu_blk, scale,
                    causal=False, window=0):
    """softmax(scale * Q K^T) V of each block over its [context; block] keys.

    ``q`` ``[T, Hq, Dh]``, ``k_blk``/``v_blk`` ``[T, Hkv, Dh]`` (already normed
    and rotated for q and k), ``k_ctx``/``v_ctx`` ``[sum C, Hkv, Dh]``;
    ``cu_ctx``/``cu_blk`` are the ``[R+1]`` cumulative row counts. Returns the
    block-query outputs ``[T, Hq, Dh]``.

    "qwen3_dflash.cpp" page, ``ForwardWithCtxKVDev``: each request's combined
    sequence is its context rows followed by its block rows, the attention runs
    over it with the layer's causal / window flags, and only the block-query
    rows are kept; scale is 1/sqrt(head_dim).
    """
    q = _f64(q)
    k_blk = _f64(k_blk)
    v_blk = _f64(v_blk)
    k_ctx = _f64(k_ctx)
    v_ctx = _f64(v_ctx)
    cu_ctx = np.asarray(cu_ctx, dtype=np.int64)
    cu_blk = np.asarray(cu_blk, dtype=np.int64)
    t, hq, d = q.shape
    hkv = k_blk.shape[1]
    group = hq // hkv
    out = np.zeros((t, hq, d), dtype=np.float64)
    for r in range(len(cu_blk) - 1):
        c0, c1 = cu_ctx[r], cu_ctx[r + 1]
        b0, b1 = cu_blk[r], cu_blk[r + 1]
        if b1 == b0:
            continue
        keys = np.concatenate([k_ctx[c0:c1], k_blk[b0:b1]], axis=0)
        vals = np.concatenate([v_ctx[c0:c1], v_blk[b0:b1]], axis=0)
        vis = attention_visibility(int(c1 - c0), int(b1 - b0), causal, window)
        for h in range(hq):
            g = h // group
            s = scale * (q[b0:b1, h, :] @ keys[:, g, :].T)
            s = np.where(vis, s, -np.inf)
            m = np.max(s, axis=1, keepdims=True)
            m = np.where(np.isfinite(m), m, 0.0)
            e = np.where(vis, np.exp(s - m), 0.0)
            denom = e.sum(axis=1, keepdims=True)
            num = e @ vals[:, g, :]
            out[b0:b1, h, :] = np.where(denom > 0, num / np.where(denom > 0, denom, 1.0), 0.0)
    return out


def draft_block_attention(q, k_blk, v_blk, blk_positions, k_ctx_hat, v_ctx,
                          cu_ctx, cu_blk, q_norm_w, k_norm_w, eps, theta,
                          scale, causal=False, window=0):
    """The whole draft-side path for one layer: q/k norm -> RoPE -> attention.

    Block q and k are raw projections; the context keys ``k_ctx_hat`` are
    already normed and rotated (the output of ``context_kv`` or of the K-only
    ``qk_norm_rope``). Returns ``(out, q_hat, k_blk_hat)``.

    "qwen3_dflash.cpp" page, ``ForwardWithCtxKVDev``: q/k RMSNorm, RopeNeox,
    then block attention over [context; block].
    """
    q_hat, k_hat = qk_norm_rope(q, k_blk, q_norm_w, k_norm_w, blk_positions, eps, theta)
    out = block_attention(q_hat, k_hat, v_blk, k_ctx_hat, v_ctx, cu_ctx, cu_blk,
                          scale, causal, window)
    return out, q_hat, k_hat


def paged_context_rows(pool, block_table, ctx_lens, page_size=16):
    """The packed context rows a paged store holds: for request r and context
    row k < ctx_lens[r], row pool[block_table[r][k // page_size], k % page_size]
    ("qwen3_dflash.cpp" page, the paged draft-KV store). ``pool`` is
    [pages, page_size, ...]; requests are concatenated in order."""
    pool = np.asarray(pool)
    block_table = np.asarray(block_table)
    rows = []
    for r, c in enumerate(np.asarray(ctx_lens).tolist()):
        for k in range(int(c)):
            rows.append(pool[int(block_table[r][k // page_size]), k % page_size])
    if not rows:
        return np.zeros((0,) + pool.shape[2:], dtype=pool.dtype)
    return np.stack(rows)


def residual_rms_norm(hidden, residual, w, eps):
    """The layer's input norm: ``res = hidden + residual`` (``hidden`` alone when
    ``residual`` is None), then ``normed = RMSNorm(res, w)``. Returns
    ``(res, normed)``.

    "qwen3_dflash.cpp" page, ``ForwardBlockLogits`` / ``ForwardWithCtxKVDev``:
    input_layernorm is the standard add + RMSNorm (the norm of hidden plus the
    residual stream, which is updated to that sum).
    """
    h = _f64(hidden)
    res = h if residual is None else h + _f64(residual)
    return res, rms_norm(res, w, eps)


def block_qkv(normed, w_qkv, num_q_heads, num_kv_heads, head_dim):
    """Merged q/k/v projection of the block rows: ``qkv = normed @ w_qkv.T``.

    ``w_qkv`` is ``[(Hq + 2 Hkv) * Dh, H]``; its rows are the q heads, then
    the k heads, then the v heads, each head Dh consecutive rows. Returns raw
    ``q [T, Hq, Dh]``, ``k [T, Hkv, Dh]``, ``v [T, Hkv, Dh]``.

    "qwen3_dflash.cpp" page, ``ForwardBlockLogits``: one product against the
    merged weight, then the split into q, k and v (the unmerged form takes the
    row slices [0, qdim), [qdim, qdim + kdim), [qdim + kdim, qdim + 2 kdim)).
    """
    qkv = _f64(normed) @ _f64(w_qkv).T
    t = qkv.shape[0]
    qd = num_q_heads * head_dim
    kd = num_kv_heads * head_dim
    q = qkv[:, :qd].reshape(t, num_q_heads, head_dim)
    k = qkv[:, qd:qd + kd].reshape(t, num_kv_heads, head_dim)
    v = qkv[:, qd + kd:qd + 2 * kd].reshape(t, num_kv_heads, head_dim)
    return q, k, v


def output_projection(attn, w_o):
    """o_proj: each row's attention output ``[Hq, Dh]`` read as one vector of
    Hq * Dh (head-major), times ``w_o.T`` (``w_o`` is ``[H, Hq * Dh]``).

    "qwen3_dflash.cpp" page, ``ForwardBlockLogits`` / ``ForwardWithCtxKVDev``:
    the attention output reshaped to ``[T, Hq * Dh]`` and multiplied by the
    o_proj weight (MatmulBT).
    """
    a = _f64(attn)
    return a.reshape(a.shape[0], -1) @ _f64(w_o).T


def draft_layer_attention(hidden, residual, in_norm_w, w_qkv, w_o, blk_positions,
                          k_ctx_hat, v_ctx, cu_ctx, cu_blk, q_norm_w, k_norm_w,
                          num_q_heads, num_kv_heads, head_dim, eps, theta, scale,
                          causal=False, window=0):
    """The draft layer's attention block: input_layernorm (residual add +
    RMSNorm), merged q/k/v projection, q/k norm + RoPE, block attention over
    [context; block], o_proj. Returns ``(o, res, q, k, v, attn)`` with q, k,
    v the raw projections.

    "qwen3_dflash.cpp" page, ``ForwardWithCtxKVDev``, in that order.
    """
    res, normed = residual_rms_norm(hidden, residual, in_norm_w, eps)
    q, k, v = block_qkv(normed, w_qkv, num_q_heads, num_kv_heads, head_dim)
    attn, _, _ = draft_block_attention(q, k, v, blk_positions, k_ctx_hat, v_ctx, cu_ctx, cu_blk,
                                       q_norm_w, k_norm_w, eps, theta, scale, causal, window)
    return output_projection(attn, w_o), res, q, k, v, attn


PAD_SLOT = -1  # slot of padding rows ("runner.cpp" page: vLLM's pad slot id)


def prepare_dflash_inputs(idx_mapping, target_query_start_loc, target_positions, num_rejected,
                          num_sampled, last_sampled, next_prefill_tokens, block_table,
                          num_query_per_req, num_speculative_steps, block_size, max_num_reqs,
                          max_num_tokens, max_model_len, mask_token_id, sample_from_anchor):
    """Integer preparation of one DFlash propose step (plain Python loops).

    "qwen3_dflash.cpp" page, ``PrepareDflashInputs`` (the host form of the
    speculator's input-preparation kernel): per request r, the verified
    target tokens of the step are its context rows; the last ``num_rejected``
    of them are rolled back, so the block (the anchor token -- the bonus token
    last sampled, or the next prefill token for a request that sampled
    nothing -- followed by mask tokens) starts right after the last kept
    position. Context and block rows get KV slots from the request's block
    table (page = position // block_size, clamped to the last page; slot =
    page id * block_size + position % block_size). The sampled rows of each
    request are its block rows from offset 0 (``sample_from_anchor``) or 1.
    Unused tail entries are padded (query_start_loc with the last end,
    seq_lens 0, sample maps 0 / 0 / -1, query slots PAD_SLOT). ``ctx_cu`` is the
    running sum of the kept context lengths (last kept position + 1) over the
    requests -- the cumulative context offsets the "runner.cpp" page hands
    the block forward (``ctx_cu``) -- padded with its total.

    Returns a dict of int64 numpy arrays.
    """
    nreq = len(idx_mapping)
    nqpr, nspec, bs = int(num_query_per_req), int(num_speculative_steps), int(block_size)
    tqsl = [int(x) for x in target_query_start_loc]
    tpos = [int(x) for x in target_positions]
    bt = np.asarray(block_table, dtype=np.int64).reshape(nreq, -1)
    stride = bt.shape[1]
    ntgt = tqsl[nreq]
    out = {
        "input_ids": np.zeros(nreq * nqpr, np.int64),
        "query_positions": np.zeros(nreq * nqpr, np.int64),
        "query_start_loc": np.zeros(max_num_reqs + 1, np.int64),
        "seq_lens": np.zeros(max_num_reqs, np.int64),
        "query_slot_mapping": np.zeros(max_num_tokens, np.int64),
        "context_positions": np.zeros(ntgt, np.int64),
        "context_slot_mapping": np.zeros(ntgt, np.int64),
        "sample_indices": np.zeros(max_num_reqs * nspec, np.int64),
        "sample_pos": np.zeros(max_num_reqs * nspec, np.int64),
        "sample_idx_mapping": np.zeros(max_num_reqs * nspec, np.int64),
        "ctx_cu": np.zeros(max_num_reqs + 1, np.int64),
    }

    def slot(r, pos):
        page = min(pos // bs, stride - 1)
        return int(bt[r, page]) * bs + pos % bs

    first_sample = 0 if sample_from_anchor else 1
    for r in range(nreq):
        state = int(idx_mapping[r])
        start, end = tqsl[r], tqsl[r + 1]
        kept_end = end - int(num_rejected[r])          # rollback of rejected drafts
        anchor = int(last_sampled[state]) if int(num_sampled[r]) > 0 else int(next_prefill_tokens[state])
        last_kept = tpos[kept_end - 1]
        for t in range(start, end):                    # the step's target rows: context
            out["context_positions"][t] = tpos[t]
            out["context_slot_mapping"][t] = slot(r, tpos[t])
        for off in range(nqpr):                        # the block: anchor + mask tokens
            pos = last_kept + 1 + off
            qi = r * nqpr + off
            out["input_ids"][qi] = anchor if off == 0 else mask_token_id
            out["query_positions"][qi] = min(pos, max_model_len - 1)
            out["query_slot_mapping"][qi] = slot(r, pos)
            if off >= first_sample:
                si = r * nspec + off - first_sample
                out["sample_indices"][si] = qi
                out["sample_pos"][si] = pos + 1 if sample_from_anchor else pos
                out["sample_idx_mapping"][si] = state
        out["query_start_loc"][r] = r * nqpr
        out["seq_lens"][r] = last_kept + 1 + nqpr
        out["ctx_cu"][r + 1] = out["ctx_cu"][r] + last_kept + 1
    for i in range(nreq, max_num_reqs + 1):
        out["query_start_loc"][i] = nreq * nqpr
        out["ctx_cu"][i] = out["ctx_cu"][nreq]
    for i in range(nreq * nspec, max_num_reqs * nspec):
        out["sample_idx_mapping"][i] = -1
    for i in range(nreq * nqpr, max_num_tokens):
        out["query_slot_mapping"][i] = PAD_SLOT
    return out


def fc_combine(aux, w_fc):
    """Multi-tap feature combine: the target's tapped hidden states
    ``aux [T, H * taps]`` rounded to bf16, times ``w_fc [H, H * taps]`` (as
    x W^T). "qwen3_dflash.cpp" page, ``CombineAuxFeatures`` (f32 aux cast to
    bf16, then the fc MatmulBT). ``aux`` is taken as given; the bf16 rounding
    of f32 inputs is the caller's (see ``bf16_round``)."""
    return _f64(aux) @ _f64(w_fc).T


def bf16_round(x):
    """Round float values to the nearest bfloat16 (ties to even), as float64:
    the f32 -> bf16 cast of ``CombineAuxFeatures`` ("qwen3_dflash.cpp" page)."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)
