/*
 * dflash.h -- C ABI of libdflash: the DFlash draft model's block attention on
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed. On the "qwen3_dflash.cpp" page (file header,
 * ForwardWithCtxKVDev, ForwardPagedBody) each speculative block of B query
 * tokens of a request attends over that request's C precomputed context K/V
 * rows followed by the block's own K/V rows. Full-attention layers see the
 * whole [context; block] sequence (bidirectional inside the block); sliding
 * window layers are causal with a window. Heads use grouped-query attention;
 * q and k get a per-head RMSNorm and a NeoX rotary embedding before the
 * attention. The context rows come from the hidden-state RMSNorm, the K/V
 * projection, the per-head k-norm and RoPE (PrecomputeContextKVDevice).
 *
 * Conventions shared by every call.
 *   - All tensor pointers are DEVICE pointers unless stated otherwise; all
 *     tensors are dense row-major with no padding, and 16-byte aligned.
 *   - "bf16" is bfloat16 (round to nearest even on every store); "f32" is IEEE
 *     binary32. Arithmetic is f32 in every kernel (bf16 matrix-core products
 *     accumulate in f32).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Every
 *     call only enqueues work on it: no host synchronisation, no allocation,
 *     so the calls may be captured into a HIP graph (the DFLASH_VALIDATE debug
 *     mode below is the one exception).
 *   - The caller owns every buffer (inputs, outputs, workspaces). The library
 *     keeps no state between calls.
 *   - Errors: a call returns a negative dflash_status and leaves a message for
 *     dflash_last_error() (per thread). Argument errors are detected on the
 *     host before anything is enqueued. Integer metadata that lives on the
 *     device (cumulative lengths, positions) is trusted to be consistent with
 *     the host-side sizes; kernels clamp every index they derive from it to the
 *     buffers' extents, so inconsistent metadata gives wrong results, never an
 *     out-of-bounds access.
 *   - Debug mode: with the environment variable DFLASH_VALIDATE set to a value
 *     other than "" or "0" (read at every call), the calls that take integer
 *     metadata on the device first copy it to the host on their stream, wait
 *     for it, and return DFLASH_ERR_INVALID_ARG, naming the first offending
 *     entry, before anything is enqueued if it breaks a precondition that the
 *     pages check on the host: block attention (all three forms): cumulative
 *     lengths start at 0, never decrease, end at total_ctx / total_blk, no
 *     request has more than max_blk_len block rows, and they equal the host
 *     copies when those are given; the fused prologue's positions lie in
 *     [0, max_pos); over a paged store, every page a request's context needs
 *     fits max_pages_per_req and its id lies in [0, num_pages).
 *     dflash_qk_norm_rope and dflash_context_kv: positions in [0, max_pos).
 *     dflash_kv_scatter: no two rows write the same slot. This mode waits for
 *     the stream, so on a stream that is being captured these calls return
 *     DFLASH_ERR_UNSUPPORTED.
 *
 * Head geometry: Hq query heads, Hkv key/value heads (Hq % Hkv == 0), head
 * dimension Dh in {64, 128}. q-head h reads kv-head h / (Hq / Hkv).
 */
#ifndef DFLASH_H_
#define DFLASH_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DFLASH_OK = 0,
  DFLASH_ERR_INVALID_ARG = -1, /* bad size, pointer, alignment or flag */
  DFLASH_ERR_UNSUPPORTED = -2, /* valid but not implemented (e.g. Dh = 96) */
  DFLASH_ERR_WORKSPACE = -3,   /* workspace missing, misaligned or too small */
  DFLASH_ERR_HIP = -4          /* the HIP runtime reported an error */
} dflash_status;

/* The two range markers are not data types: they make every 32-bit value a
 * valid dflash_dtype in C++ as in C, so that the library can reject any value
 * a caller passes (DFLASH_ERR_INVALID_ARG) without reading an out-of-range
 * enumeration value. */
typedef enum {
  DFLASH_F32 = 0,
  DFLASH_BF16 = 1,
  DFLASH_DTYPE_RANGE_MIN_ = -0x7fffffff - 1,
  DFLASH_DTYPE_RANGE_MAX_ = 0x7fffffff
} dflash_dtype;

/* Message of the last failed call on this thread ("" if none). Never NULL. */
const char* dflash_last_error(void);

/* ABI version of this header (major * 100 + minor). */
int dflash_abi_version(void);

/*
 * dflash_rope_table -- the NeoX rotary cos/sin cache.
 *
 * Fills table[p][i] = {cos(p * f_i), sin(p * f_i)} for p in [0, max_pos) and
 * i in [0, head_dim / 2), with f_i = theta^(-2 i / head_dim); angles, cos and
 * sin are evaluated in f64 and rounded once to f32. This is the cos|sin cache
 * the "qwen3.cpp" page (file header) keeps for RoPE; the rotation itself is
 * RopeNeox on the "qwen3_dflash.cpp" page.
 *
 *   table    device f32, max_pos * head_dim elements (pairs), written.
 *   max_pos  >= 1; head_dim even, 2..256; theta > 0.
 */
dflash_status dflash_rope_table(float* table, int32_t max_pos, int32_t head_dim, double theta,
                                void* stream);

/*
 * dflash_qk_norm_rope -- per-head RMSNorm of q and k, then NeoX RoPE, in place.
 *
 * For every row t and head h of q [T, Hq, Dh] and k [T, Hkv, Dh]:
 *   y = x * w / sqrt(mean(x^2) + eps)           (w = q_norm_w or k_norm_w)
 *   (y_i, y_{i+Dh/2}) <- (y_i c - y_{i+Dh/2} s, y_{i+Dh/2} c + y_i s)
 * with (c, s) = rope_table[positions[t]][i]. "qwen3_dflash.cpp" page,
 * ForwardBlockLogits: q_norm and k_norm (standard RMSNorm over head_dim), then
 * RopeNeox at the block positions; "qwen3.cpp" page header: norm before RoPE.
 *
 *   dtype      DFLASH_BF16 or DFLASH_F32, for q and k.
 *   q          [T, Hq, Dh] in/out, or NULL for the K-only form (context rows).
 *   k          [T, Hkv, Dh] in/out (not NULL).
 *   q_norm_w   f32 [Dh] (ignored when q is NULL), k_norm_w f32 [Dh].
 *   positions  int32 [T]; a position outside [0, max_pos) is clamped into it.
 *   rope_table f32 [max_pos][Dh/2][2] from dflash_rope_table.
 *   T may be 0 (nothing is enqueued).
 */
dflash_status dflash_qk_norm_rope(dflash_dtype dtype, void* q, void* k, const float* q_norm_w,
                                  const float* k_norm_w, const int32_t* positions, int64_t T,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  float eps, const float* rope_table, int32_t max_pos,
                                  void* stream);

/*
 * Block attention parameters (host values). Mirrors the arguments of the
 * block attention call on the "qwen3_dflash.cpp" page ({scale, causal,
 * sliding_window, cu_seqlens, num_reqs}) with the context and block rows given
 * as two separate packed sources instead of one materialised sequence.
 */
typedef struct {
  int32_t num_reqs;     /* R >= 1 */
  int32_t num_q_heads;  /* Hq */
  int32_t num_kv_heads; /* Hkv, divides Hq */
  int32_t head_dim;     /* Dh in {64, 128} */
  dflash_dtype dtype;   /* of q, k_*, v_*, out */
  int64_t total_ctx;    /* rows of k_ctx / v_ctx (= cu_ctx_lens[R]) */
  int64_t total_blk;    /* rows of q / k_blk / v_blk / out (= cu_blk_lens[R]) */
  int32_t max_blk_len;  /* upper bound on any request's block length */
  float scale;          /* softmax scale, 1/sqrt(Dh) on the pages */
  int32_t causal;       /* 0: bidirectional, else causal */
  int32_t window;       /* 0: none; > 0 (causal only): keys with i - k < window */
  int32_t split_keys;   /* keys per work unit; 0 = chosen by the library,
                           else a positive multiple of 64 */
  /* Optional HOST copies of cu_ctx_lens / cu_blk_lens (int32 [R+1] each, equal
   * to the device arrays; both or neither). With them the split of the keys
   * into work units is planned on the host and handed to the kernels with the
   * launch (up to 64 requests, 512 units per kv-head and 256 per request;
   * beyond that, and when NULL, the kernels plan it from the device arrays;
   * the result is bitwise the same either way). The bf16 kernels then take
   * the row ranges from these copies (the f32 path always reads the device
   * arrays). They are read during the call only; under stream capture the
   * plan is fixed into the graph, so the lengths must not change between
   * replays. Checked: [0] = 0, nondecreasing, cu_ctx_lens[R] = total_ctx,
   * cu_blk_lens[R] = total_blk, block lengths <= max_blk_len. The pages build
   * the same per-request offsets on the host ("qwen3_dflash.cpp" page,
   * ForwardWithCtxKVDev: cu_comb and the index maps from host vectors). */
  const int32_t* host_cu_ctx_lens;
  const int32_t* host_cu_blk_lens;
} dflash_block_attn_params;

/*
 * Optional fused prologue of dflash_block_attention: when given, q and k_blk
 * are the RAW projections and the attention applies, on the fly, exactly
 * what dflash_qk_norm_rope would (per-head RMSNorm with q_norm_w / k_norm_w,
 * then NeoX RoPE at `positions`), without writing q or k_blk back
 * ("qwen3_dflash.cpp" page, ForwardBlockLogits: q_norm, k_norm, RopeNeox right
 * before the block attention; "qwen3.cpp" page header names this fusion
 * kAttnQkNormRope). Requires dtype == DFLASH_BF16 and max_blk_len <= 64
 * (DFLASH_ERR_UNSUPPORTED otherwise).
 */
typedef struct {
  const float* q_norm_w;    /* device f32 [Dh] */
  const float* k_norm_w;    /* device f32 [Dh] */
  const int32_t* positions; /* device int32 [total_blk]: positions of the block rows,
                               clamped into [0, max_pos) */
  const float* rope_table;  /* device f32 [max_pos][Dh/2][2] from dflash_rope_table */
  int32_t max_pos;
  float eps;
} dflash_qk_prologue;

/* Bytes of workspace dflash_block_attention needs for these parameters
 * (0 if they are invalid; see dflash_block_attention_check). */
size_t dflash_block_attention_workspace_size(const dflash_block_attn_params* p);

/* Host-side validation only: the status dflash_block_attention would return
 * for these parameters before touching any pointer. */
dflash_status dflash_block_attention_check(const dflash_block_attn_params* p);

/*
 * dflash_block_attention -- softmax(scale Q K^T) V of each block over its
 * request's [context; block] keys.
 *
 * Request r owns context rows [cu_ctx_lens[r], cu_ctx_lens[r+1]) of k_ctx/v_ctx
 * and block rows [cu_blk_lens[r], cu_blk_lens[r+1]) of q/k_blk/v_blk/out. In
 * its combined sequence the context rows take indices 0..C-1 and the block rows
 * C..C+B-1; block query b sits at index C+b. Key k is visible to it always
 * (causal == 0), or iff k <= C+b and (window == 0 or C+b-k < window). Only block
 * queries are computed ("qwen3_dflash.cpp" page, ForwardWithCtxKVDev keeps only
 * the block rows of the combined attention; ForwardPagedBody computes them
 * directly).
 *
 *   cu_ctx_lens, cu_blk_lens  device int32 [R+1], nondecreasing, [0] = 0.
 *   prologue  NULL, or the fused q/k norm + RoPE (see dflash_qk_prologue).
 *   q       [total_blk, Hq, Dh]  (already q-normed and rotated unless prologue)
 *   k_blk   [total_blk, Hkv, Dh] (already k-normed and rotated unless prologue),
 *           v_blk alike (raw).
 *   k_ctx   [total_ctx, Hkv, Dh], v_ctx alike; may be NULL if total_ctx == 0.
 *   out     [total_blk, Hq, Dh], written (rows of empty requests untouched).
 *   workspace  device, 256-byte aligned, >= dflash_block_attention_workspace_size
 *           bytes (no initialisation needed). It holds the partial results of
 *           key ranges that were split across work units (each split's
 *           softmax output scaled per query row by a power of two into fp16,
 *           with its max, sum and scale exponent in f32, so any finite bf16
 *           V fits); one workspace must not be used by two calls that may run
 *           concurrently. Products and sums accumulate in f32, which bounds
 *           |V| by about 2^100 (far beyond any activation).
 * The result does not depend on how the keys are split into work units other
 * than through f32 rounding; for a fixed split_keys it is bitwise
 * deterministic.
 */
dflash_status dflash_block_attention(const dflash_block_attn_params* p,
                                     const dflash_qk_prologue* prologue /* NULL: q, k_blk normed */,
                                     const int32_t* cu_ctx_lens,
                                     const int32_t* cu_blk_lens, const void* q, const void* k_blk,
                                     const void* v_blk, const void* k_ctx, const void* v_ctx,
                                     void* out, void* workspace, size_t workspace_bytes,
                                     void* stream);

/*
 * dflash_block_attention_noalloc -- dflash_block_attention for callers that
 * cannot allocate device memory (code under HIP-graph capture, tight serving
 * loops, harnesses that forbid allocation): the same computation, arguments
 * and result (bitwise, for the same parameters) with the workspace taken from
 * a scratch array the library holds on each GPU instead of a caller buffer.
 *
 * The scratch is DFLASH_NOALLOC_SCRATCH_BYTES (32 MiB) per GPU, held until
 * the process ends; it covers every batch whose
 * dflash_block_attention_workspace_size is at most that (e.g. 64 requests of
 * up to 8192 context rows with 16-row blocks, Hq 32, Hkv 8, Dh 128: 17 MiB).
 * Larger workspaces are rejected with DFLASH_ERR_WORKSPACE before anything is
 * enqueued. Nothing in the scratch needs to start at zero (every partial is
 * written before it is read within a call). All calls on one GPU share that
 * GPU's scratch: calls that may overlap on one GPU (on different streams, or
 * from different threads without ordering) race and must not be issued. The
 * first call on a device looks up the scratch's device address (a host-side
 * query, not a stream operation); the call itself allocates nothing.
 */
#define DFLASH_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
dflash_status dflash_block_attention_noalloc(const dflash_block_attn_params* p,
                                             const dflash_qk_prologue* prologue,
                                             const int32_t* cu_ctx_lens,
                                             const int32_t* cu_blk_lens, const void* q,
                                             const void* k_blk, const void* v_blk,
                                             const void* k_ctx, const void* v_ctx, void* out,
                                             void* stream);

/*
 * Paged context store ("qwen3_dflash.cpp" page, the fixed-capacity paged
 * draft-KV store read by the paged block attention in ForwardPagedBody): a
 * pool [num_pages, page_size, Hkv, Dh] per tensor (K and V), and per request
 * a row of block_table listing the pages of its context rows in order:
 * context row k of request r lives at pool page block_table[r * stride +
 * k / page_size], row k % page_size. Page indices past the table row and page
 * ids outside [0, num_pages) are clamped into range (wrong values, never an
 * out-of-bounds access).
 */
typedef struct {
  const int32_t* block_table;  /* device int32 [num_reqs][max_pages_per_req] */
  int32_t max_pages_per_req;   /* row stride of block_table, >= 1 */
  int32_t page_size;           /* rows per page; 16 */
  int64_t num_pages;           /* pages in each pool, >= 1 */
} dflash_paged_ctx;

/*
 * dflash_block_attention_paged -- dflash_block_attention with the context
 * K/V read from a paged store instead of packed rows.
 *
 * Identical semantics, arguments and workspace to dflash_block_attention
 * except: k_pool / v_pool are [num_pages, 16, Hkv, Dh] pools addressed through
 * pg->block_table; cu_ctx_lens still gives each request's context length
 * (C_r = cu_ctx_lens[r+1] - cu_ctx_lens[r], the pages' seq_lens) and
 * p->total_ctx = cu_ctx_lens[R]. The work split is the packed call's for the
 * same lengths whenever that split has at most 16384 keys per work unit (then
 * the result is bitwise the packed call's); longer splits are cut to that
 * size (split_keys, if given, must not exceed it). Requires page_size == 16
 * (DFLASH_ERR_UNSUPPORTED otherwise). The workspace is sized by
 * dflash_block_attention_paged_workspace_size (>= the packed size).
 */
dflash_status dflash_block_attention_paged(const dflash_block_attn_params* p,
                                           const dflash_paged_ctx* pg,
                                           const dflash_qk_prologue* prologue,
                                           const int32_t* cu_ctx_lens,
                                           const int32_t* cu_blk_lens, const void* q,
                                           const void* k_blk, const void* v_blk,
                                           const void* k_pool, const void* v_pool, void* out,
                                           void* workspace, size_t workspace_bytes,
                                           void* stream);

/* Bytes of workspace dflash_block_attention_paged needs (0 if invalid). */
size_t dflash_block_attention_paged_workspace_size(const dflash_block_attn_params* p);

/*
 * dflash_kv_scatter -- append rows to a paged store: for every row t with
 * 0 <= slot_mapping[t] < num_slots, pool row slot_mapping[t] of k_pool and
 * v_pool (a flat view [num_slots, Hkv, Dh], slot = page * page_size + offset)
 * receives row t of k_src and v_src; other rows (e.g. the padding slot -1)
 * are skipped. The pages' store appends context rows this way (an index copy
 * to slots). Rows with equal slots race (the caller gives distinct slots).
 *
 *   dtype        of every tensor; k_src, v_src [T, Hkv, Dh]; slot_mapping int32 [T].
 *   T may be 0 (nothing is enqueued).
 */
dflash_status dflash_kv_scatter(dflash_dtype dtype, const void* k_src, const void* v_src,
                                const int32_t* slot_mapping, int64_t T, int32_t num_kv_heads,
                                int32_t head_dim, void* k_pool, void* v_pool, int64_t num_slots,
                                void* stream);

/*
 * dflash_context_kv -- context K/V precompute (bf16).
 *
 * For each context row t: n = RMSNorm(hidden[t], hidden_norm_w); K = n W_k^T,
 * V = n W_v^T; K <- per-head RMSNorm(K, k_norm_w); K <- NeoX RoPE at
 * positions[t]; V stays raw. "qwen3_dflash.cpp" page,
 * PrecomputeContextKVDevice (W_k and W_v are the K and V row slices of the
 * merged qkv weight; the result is the ContextKVDev record).
 *
 *   hidden        bf16 [T, H]
 *   hidden_norm_w f32 [H];  w_k, w_v bf16 [Hkv*Dh, H];  k_norm_w f32 [Dh]
 *   positions     int32 [T], clamped into [0, max_pos)
 *   rope_table    f32 [max_pos][Dh/2][2] from dflash_rope_table
 *   k_out, v_out  bf16 [T, Hkv, Dh], written
 *   workspace     device, 256-byte aligned, >= dflash_context_kv_workspace_size
 *                 bytes (no zero-fill needed)
 * Requirements: Dh == 128, H % 64 == 0, (Hkv * Dh) % 256 == 0, H and Hkv * Dh
 * at most 2^20 (the workspace-size query returns 0 beyond). Calls of at
 * least 256 rows fold the norm weight into the weights and run one fused
 * GEMM + k-norm + RoPE kernel; calls of fewer rows (a propose step appending
 * its verified rows) round the normed rows to bf16, run the split-K projection
 * GEMM and then the k-norm + RoPE (and need H <= 8192). Each output row
 * depends only on its own input row: splitting the rows across calls of at
 * least 256 rows each gives bitwise identical results. Calls of fewer rows
 * sum the partials of a split over H whose slice count follows from the
 * number of 128-row tiles (at H = 4096 and Hkv = 8: 8 slices for up to 128
 * rows, 4 for 129 to 255), so such calls give identical bits when they plan
 * the same split; all forms agree within bf16 rounding.
 */
size_t dflash_context_kv_workspace_size(int64_t T, int32_t hidden_size, int32_t num_kv_heads,
                                        int32_t head_dim);
dflash_status dflash_context_kv(const void* hidden, const float* hidden_norm_w, const void* w_k,
                                const void* w_v, const float* k_norm_w, const int32_t* positions,
                                int64_t T, int32_t hidden_size, int32_t num_kv_heads,
                                int32_t head_dim, float eps, const float* rope_table,
                                int32_t max_pos, void* k_out, void* v_out, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * dflash_block_qkv -- the draft layer's input norm and merged q/k/v
 * projection of the block rows (bf16).
 *
 * For each block row t: res = hidden[t] + residual[t] (rounded to bf16 and
 * written back to residual; with residual == NULL, res = hidden[t] and nothing
 * is written), n = bf16(RMSNorm(res, norm_w)), qkv = n W_qkv^T, split into
 * q | k | v by column: columns [0, Hq Dh) are q, the next Hkv Dh are k, the
 * last Hkv Dh are v. q and k are the raw projections: the q/k RMSNorm and
 * RoPE are the attention's fused prologue (dflash_qk_prologue) or
 * dflash_qk_norm_rope. "qwen3_dflash.cpp" page, ForwardBlockLogits /
 * ForwardWithCtxKVDev (input_layernorm as the standard add + RMSNorm, the
 * merged qkv weight as one product, then the q/k/v split).
 *
 *   hidden     bf16 [T, H];  residual bf16 [T, H] (in/out) or NULL
 *   norm_w     f32 [H] (the input_layernorm weight)
 *   w_qkv      bf16 [(Hq + 2 Hkv) Dh, H], row-major (rows: q heads, k heads, v heads)
 *   q          bf16 [T, Hq, Dh];  k, v bf16 [T, Hkv, Dh] (written)
 *   workspace  device, 256-byte aligned, >= dflash_block_qkv_workspace_size
 *              bytes (no zero-fill needed): the normed rows and, for small T,
 *              f32 partial products of a split over H
 * Requirements: Dh in {64, 128}, Hq % Hkv == 0, H % 64 == 0, H <= 8192; all
 * tensors 16-byte aligned. T may be 0 (nothing is enqueued). Rows are
 * independent. The caller owns every buffer; the call is asynchronous on
 * `stream` and allocates nothing.
 */
size_t dflash_block_qkv_workspace_size(int64_t T, int32_t hidden_size, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim);
dflash_status dflash_block_qkv(const void* hidden, void* residual, const float* norm_w,
                               const void* w_qkv, int64_t T, int32_t hidden_size,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               float eps, void* q, void* k, void* v, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * dflash_o_proj -- the draft layer's output projection (bf16).
 *
 * out[t] = attn[t] W_o^T, where attn[t] is the attention output row [Hq, Dh]
 * read as one vector of in_dim = Hq Dh (head-major) and W_o is [H, in_dim].
 * "qwen3_dflash.cpp" page, ForwardBlockLogits / ForwardWithCtxKVDev (o_proj
 * applied to the attention output reshaped to [T, Hq Dh]).
 *
 *   attn       bf16 [T, in_dim];  w_o bf16 [H, in_dim];  out bf16 [T, H] (written)
 *   workspace  device, 256-byte aligned, >= dflash_o_proj_workspace_size bytes
 *              (may be 0 bytes and NULL when that is 0)
 * Requirements: H % 64 == 0, in_dim % 64 == 0; tensors 16-byte aligned. T may
 * be 0.
 */
size_t dflash_o_proj_workspace_size(int64_t T, int32_t hidden_size, int32_t in_dim);
dflash_status dflash_o_proj(const void* attn, const void* w_o, int64_t T, int32_t hidden_size,
                            int32_t in_dim, void* out, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * dflash_prepare_inputs -- integer preparation of one propose step.
 *
 * "qwen3_dflash.cpp" page, PrepareDflashInputs. Per request r (state s =
 * idx_mapping[r]): the step's target rows [start, end) =
 * target_query_start_loc[r .. r+1] are context rows (their positions and KV
 * slots are written); the last num_rejected[r] of them are rolled back, so the
 * block of num_query_per_req rows (the anchor -- last_sampled[s] if
 * num_sampled[r] > 0, else next_prefill_tokens[s] -- then mask_token_id)
 * takes positions last_kept + 1 + off (query_positions clamped to
 * max_model_len - 1; slots from the unclamped position). A slot is
 * block_table[r][min(pos / block_size, stride - 1)] * block_size +
 * pos % block_size. Block row off >= (sample_from_anchor ? 0 : 1) is sampled:
 * sample_indices / sample_pos (pos + 1 when sampling from the anchor, else
 * pos) / sample_idx_mapping (= s) at r * num_speculative_steps + off - first.
 * query_start_loc[r] = r * nqpr, seq_lens[r] = last_kept + 1 + nqpr, and the
 * cumulative kept-context lengths ctx_cu[r + 1] = ctx_cu[r] + last_kept + 1
 * (ctx_cu[0] = 0; the runner page's ctx_cu, the attention's cu_ctx_lens, with
 * query_start_loc as its cu_blk_lens). Tails: query_start_loc[R ..
 * max_num_reqs] = R * nqpr, ctx_cu[R + 1 .. max_num_reqs] = ctx_cu[R],
 * seq_lens[R ..) = 0, sample maps [R * nspec ..) = 0 / 0 / -1,
 * query_slot_mapping[R * nqpr .. max_num_tokens) = -1 (the pad slot).
 * Positions and slots are int32 (as every other call of this library takes
 * them); integer only: bit-exact.
 *
 * Requirements (checked): num_reqs >= 1, max_num_reqs >= num_reqs,
 * max_num_tokens >= num_reqs * nqpr, nqpr >= 1, num_speculative_steps ==
 * nqpr - (sample_from_anchor ? 0 : 1), block_size >= 1, block_table_stride >=
 * 1, max_model_len >= 1, num_states >= 1, num_target_tokens >= 1 (the host
 * copy of target_query_start_loc[num_reqs]), every pointer non-NULL.
 * Positions are >= 0. Device metadata is trusted; indices derived from it are
 * clamped into their buffers.
 */
typedef struct {
  int32_t num_reqs, max_num_reqs, max_num_tokens;
  int32_t num_query_per_req;      /* 1 + k: the anchor and k mask rows */
  int32_t num_speculative_steps;  /* sampled rows per request */
  int32_t block_size, block_table_stride;
  int32_t max_model_len, mask_token_id, sample_from_anchor;
  int32_t num_states;             /* entries of last_sampled / next_prefill_tokens */
  int64_t num_target_tokens;
} dflash_prepare_params;

typedef struct { /* device inputs */
  const int32_t* idx_mapping;             /* [num_reqs] */
  const int32_t* target_query_start_loc;  /* [num_reqs + 1] */
  const int32_t* target_positions;        /* [num_target_tokens] */
  const int32_t* num_rejected;            /* [num_reqs] */
  const int32_t* num_sampled;             /* [num_reqs] */
  const int32_t* last_sampled;            /* [num_states] */
  const int32_t* next_prefill_tokens;     /* [num_states] */
  const int32_t* block_table;             /* [num_reqs][block_table_stride] */
} dflash_prepare_inputs_in;

typedef struct { /* device outputs */
  int32_t* input_ids;             /* [num_reqs * nqpr] */
  int32_t* query_positions;       /* [num_reqs * nqpr] */
  int32_t* query_start_loc;       /* [max_num_reqs + 1] */
  int32_t* seq_lens;              /* [max_num_reqs] */
  int32_t* query_slot_mapping;    /* [max_num_tokens] */
  int32_t* context_positions;     /* [num_target_tokens] */
  int32_t* context_slot_mapping;  /* [num_target_tokens] */
  int32_t* sample_indices;        /* [max_num_reqs * nspec] */
  int32_t* sample_pos;            /* [max_num_reqs * nspec] */
  int32_t* sample_idx_mapping;    /* [max_num_reqs * nspec] */
  int32_t* ctx_cu;                /* [max_num_reqs + 1] */
} dflash_prepare_inputs_out;

dflash_status dflash_prepare_inputs(const dflash_prepare_params* p,
                                    const dflash_prepare_inputs_in* in,
                                    const dflash_prepare_inputs_out* out, void* stream);

/*
 * dflash_fc_combine -- the multi-tap feature combine (bf16 product).
 *
 * out = bf16(aux) w_fc^T: the target's tapped hidden states aux [T, H * taps]
 * (f32) rounded to bf16, times the fc weight w_fc [H, H * taps] (bf16,
 * row-major), out [T, H] bf16. "qwen3_dflash.cpp" page, CombineAuxFeatures.
 * workspace: 256-byte aligned, >= dflash_fc_combine_workspace_size bytes.
 * Requirements: H % 64 == 0, num_taps >= 1; tensors 16-byte aligned; T may be 0.
 */
size_t dflash_fc_combine_workspace_size(int64_t T, int32_t hidden_size, int32_t num_taps);
dflash_status dflash_fc_combine(const float* aux, const void* w_fc, int64_t T, int32_t hidden_size,
                                int32_t num_taps, void* out, void* workspace,
                                size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH_H_ */
