// C ABI of libdflash: argument validation, error reporting, launch dispatch.
//
// Host checks mirror the preconditions the "qwen3_dflash.cpp" page enforces
// with VT_CHECK (num_reqs > 0, cumulative lengths spanning the rows, matching
// sizes), turned into status codes plus a per-thread message instead of
// exceptions. Nothing here allocates device memory or synchronises, except in
// the DFLASH_VALIDATE debug mode (below), which copies device-resident
// metadata to the host and waits for it.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "dflash_internal.h"

namespace {

thread_local std::string g_last_error;

dflash_status fail(dflash_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

dflash_status ok() {
  g_last_error.clear();
  return DFLASH_OK;
}

dflash_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(DFLASH_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// The work split is planned for the MI355X's compute-unit count so that the
// plan (and therefore the workspace size and the bitwise result for a given
// input) is a pure function of the parameters.
constexpr int kPlanComputeUnits = 256;
constexpr int kPagedMaxUnitKeys = 16384;  // keys per work unit over a paged store

dflash_status check_head_geometry(int32_t hq, int32_t hkv, int32_t dh, bool need_q) {
  if (hkv < 1) return fail(DFLASH_ERR_INVALID_ARG, "num_kv_heads must be >= 1 (got %d)", hkv);
  if (need_q && hq < 1) return fail(DFLASH_ERR_INVALID_ARG, "num_q_heads must be >= 1 (got %d)", hq);
  if (need_q && hq % hkv != 0)
    return fail(DFLASH_ERR_INVALID_ARG, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)",
                hq, hkv);
  if (dh <= 0 || dh % 2 != 0)
    return fail(DFLASH_ERR_INVALID_ARG, "head_dim must be positive and even (got %d)", dh);
  if (dh != 64 && dh != 128)
    return fail(DFLASH_ERR_UNSUPPORTED, "head_dim %d is not supported (64 or 128)", dh);
  return DFLASH_OK;
}

// ---------------------------------------------------------------------------
// DFLASH_VALIDATE debug mode. With the environment variable set (to anything
// but "" or "0"; read at every call), the calls that take integer metadata on
// the device copy it to the host on their stream, wait for it, and check it
// before enqueueing anything: the same preconditions the reference checks on
// the host, which the kernels otherwise trust (and only clamp).
bool validate_enabled() {
  const char* v = std::getenv("DFLASH_VALIDATE");
  return v && v[0] != '\0' && std::strcmp(v, "0") != 0;
}

// n int32 values from the device into out (synchronises the stream).
dflash_status fetch_i32(const char* who, const char* what, const int32_t* dev, int64_t n,
                        std::vector<int32_t>* out, void* stream) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing((hipStream_t)stream, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone)
    return fail(DFLASH_ERR_UNSUPPORTED,
                "%s: DFLASH_VALIDATE waits for the stream and cannot run while it is captured", who);
  out->assign((size_t)n, 0);
  if (n == 0) return DFLASH_OK;
  if (!dev) return fail(DFLASH_ERR_INVALID_ARG, "%s: %s is NULL", who, what);
  hipError_t e = hipMemcpyAsync(out->data(), dev, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToHost,
                                (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess)
    return fail(DFLASH_ERR_HIP, "%s: DFLASH_VALIDATE could not read %s: HIP error %d (%s)", who, what,
                (int)e, hipGetErrorString(e));
  return DFLASH_OK;
}

// Cumulative lengths: c[0] == 0, nondecreasing, c[R] == total; optionally each
// length <= max_len and equal to the host copy.
dflash_status check_cu(const char* who, const char* what, const std::vector<int32_t>& c, int64_t total,
                       int32_t max_len, const int32_t* host) {
  const size_t r_count = c.size() - 1;
  if (c[0] != 0) return fail(DFLASH_ERR_INVALID_ARG, "%s: %s[0] = %d, expected 0", who, what, c[0]);
  for (size_t r = 0; r < r_count; ++r) {
    if (c[r + 1] < c[r])
      return fail(DFLASH_ERR_INVALID_ARG, "%s: %s decreases at request %zu (%d -> %d)", who, what, r,
                  c[r], c[r + 1]);
    if (max_len >= 0 && c[r + 1] - c[r] > max_len)
      return fail(DFLASH_ERR_INVALID_ARG, "%s: request %zu has %d rows in %s, more than %d", who, r,
                  c[r + 1] - c[r], what, max_len);
  }
  if (c[r_count] != total)
    return fail(DFLASH_ERR_INVALID_ARG, "%s: %s ends at %d, expected %lld", who, what, c[r_count],
                (long long)total);
  if (host)
    for (size_t r = 0; r <= r_count; ++r)
      if (host[r] != c[r])
        return fail(DFLASH_ERR_INVALID_ARG, "%s: device %s[%zu] = %d differs from the host copy (%d)",
                    who, what, r, c[r], host[r]);
  return DFLASH_OK;
}

dflash_status check_positions(const char* who, const int32_t* dev, int64_t n, int32_t max_pos,
                              void* stream) {
  std::vector<int32_t> pos;
  dflash_status st = fetch_i32(who, "positions", dev, n, &pos, stream);
  if (st != DFLASH_OK) return st;
  for (int64_t i = 0; i < n; ++i)
    if (pos[(size_t)i] < 0 || pos[(size_t)i] >= max_pos)
      return fail(DFLASH_ERR_INVALID_ARG, "%s: positions[%lld] = %d is outside [0, %d)", who,
                  (long long)i, pos[(size_t)i], max_pos);
  return DFLASH_OK;
}

}  // namespace

extern "C" {

const char* dflash_last_error(void) { return g_last_error.c_str(); }

int dflash_abi_version(void) { return 106; }

dflash_status dflash_rope_table(float* table, int32_t max_pos, int32_t head_dim, double theta,
                                void* stream) {
  if (!table) return fail(DFLASH_ERR_INVALID_ARG, "rope_table: table is NULL");
  if (!aligned(table, 16)) return fail(DFLASH_ERR_INVALID_ARG, "rope_table: table not 16-byte aligned");
  if (max_pos < 1) return fail(DFLASH_ERR_INVALID_ARG, "rope_table: max_pos must be >= 1");
  if (head_dim < 2 || head_dim > 256 || head_dim % 2)
    return fail(DFLASH_ERR_INVALID_ARG, "rope_table: head_dim must be even in [2, 256]");
  if (!(theta > 0.0) || !std::isfinite(theta))
    return fail(DFLASH_ERR_INVALID_ARG, "rope_table: theta must be positive and finite");
  return hip_status(dflash::launch_rope_table(table, max_pos, head_dim, theta, (hipStream_t)stream),
                    "rope_table launch");
}

dflash_status dflash_qk_norm_rope(dflash_dtype dtype, void* q, void* k, const float* q_norm_w,
                                  const float* k_norm_w, const int32_t* positions, int64_t T,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  float eps, const float* rope_table, int32_t max_pos,
                                  void* stream) {
  if (dtype != DFLASH_F32 && dtype != DFLASH_BF16)
    return fail(DFLASH_ERR_INVALID_ARG, "qk_norm_rope: unknown dtype %d", (int)dtype);
  dflash_status st = check_head_geometry(num_q_heads, num_kv_heads, head_dim, q != nullptr);
  if (st != DFLASH_OK) return st;
  if (T < 0) return fail(DFLASH_ERR_INVALID_ARG, "qk_norm_rope: T must be >= 0");
  if (!(eps >= 0.f) || !std::isfinite(eps))
    return fail(DFLASH_ERR_INVALID_ARG, "qk_norm_rope: eps must be finite and >= 0");
  if (max_pos < 1) return fail(DFLASH_ERR_INVALID_ARG, "qk_norm_rope: max_pos must be >= 1");
  if (T == 0) return ok();
  if (!k || !k_norm_w || !positions || !rope_table || (q && !q_norm_w))
    return fail(DFLASH_ERR_INVALID_ARG, "qk_norm_rope: NULL pointer argument");
  if (!aligned(k, 16) || (q && !aligned(q, 16)) || !aligned(k_norm_w, 16) ||
      (q && !aligned(q_norm_w, 16)) || !aligned(rope_table, 16))
    return fail(DFLASH_ERR_INVALID_ARG, "qk_norm_rope: tensors must be 16-byte aligned");
  if (T > (int64_t)1 << 40) return fail(DFLASH_ERR_INVALID_ARG, "qk_norm_rope: T too large");
  if (validate_enabled()) {
    st = check_positions("qk_norm_rope", positions, T, max_pos, stream);
    if (st != DFLASH_OK) return st;
  }
  return hip_status(dflash::launch_qk_norm_rope(dtype, q, k, q_norm_w, k_norm_w, positions, T,
                                                num_q_heads, num_kv_heads, head_dim, eps,
                                                rope_table, max_pos, (hipStream_t)stream),
                    "qk_norm_rope launch");
}

dflash_status dflash_block_attention_check(const dflash_block_attn_params* p) {
  if (!p) return fail(DFLASH_ERR_INVALID_ARG, "block_attention: params is NULL");
  if (p->dtype != DFLASH_F32 && p->dtype != DFLASH_BF16)
    return fail(DFLASH_ERR_INVALID_ARG, "block_attention: unknown dtype %d", (int)p->dtype);
  if (p->num_reqs < 1)
    return fail(DFLASH_ERR_INVALID_ARG, "block_attention: num_reqs must be > 0 (got %d)", p->num_reqs);
  dflash_status st = check_head_geometry(p->num_q_heads, p->num_kv_heads, p->head_dim, true);
  if (st != DFLASH_OK) return st;
  if (p->total_ctx < 0 || p->total_blk < 0)
    return fail(DFLASH_ERR_INVALID_ARG, "block_attention: total_ctx/total_blk must be >= 0");
  if (p->total_ctx > INT32_MAX / 2 || p->total_blk > INT32_MAX / 2 ||
      p->total_ctx + p->total_blk > INT32_MAX / 2)
    return fail(DFLASH_ERR_INVALID_ARG, "block_attention: total rows must be < 2^30");
  if (p->max_blk_len < 0 || p->max_blk_len > p->total_blk)
    return fail(DFLASH_ERR_INVALID_ARG, "block_attention: max_blk_len must be in [0, total_blk]");
  if (p->total_blk > 0 && p->max_blk_len < 1)
    return fail(DFLASH_ERR_INVALID_ARG, "block_attention: max_blk_len must be >= 1 when total_blk > 0");
  if ((int64_t)p->max_blk_len * (p->num_q_heads / p->num_kv_heads) > INT32_MAX / 2)
    return fail(DFLASH_ERR_INVALID_ARG, "block_attention: block too long");
  if (!std::isfinite(p->scale))
    return fail(DFLASH_ERR_INVALID_ARG, "block_attention: scale must be finite");
  if (p->window < 0) return fail(DFLASH_ERR_INVALID_ARG, "block_attention: window must be >= 0");
  if (p->window > 0 && !p->causal)
    return fail(DFLASH_ERR_INVALID_ARG,
                "block_attention: a sliding window requires causal attention");
  if (p->split_keys < 0 || p->split_keys % 64 != 0 || p->split_keys > (1 << 24))
    return fail(DFLASH_ERR_INVALID_ARG,
                "block_attention: split_keys must be 0 or a positive multiple of 64 up to 2^24");
  if (!p->host_cu_ctx_lens != !p->host_cu_blk_lens)
    return fail(DFLASH_ERR_INVALID_ARG,
                "block_attention: give both host_cu_ctx_lens and host_cu_blk_lens, or neither");
  if (p->host_cu_ctx_lens) {
    const int32_t* hc = p->host_cu_ctx_lens;
    const int32_t* hb = p->host_cu_blk_lens;
    if (hc[0] != 0 || hb[0] != 0)
      return fail(DFLASH_ERR_INVALID_ARG, "block_attention: host cu lengths must start at 0");
    for (int32_t r = 0; r < p->num_reqs; ++r) {
      if (hc[r + 1] < hc[r] || hb[r + 1] < hb[r])
        return fail(DFLASH_ERR_INVALID_ARG,
                    "block_attention: host cu lengths must be nondecreasing (request %d)", r);
      if (hb[r + 1] - hb[r] > p->max_blk_len)
        return fail(DFLASH_ERR_INVALID_ARG,
                    "block_attention: request %d has %d block rows > max_blk_len %d", r,
                    hb[r + 1] - hb[r], p->max_blk_len);
    }
    if (hc[p->num_reqs] != p->total_ctx || hb[p->num_reqs] != p->total_blk)
      return fail(DFLASH_ERR_INVALID_ARG,
                  "block_attention: host cu lengths end at %d / %d, expected total_ctx %lld / "
                  "total_blk %lld", hc[p->num_reqs], hb[p->num_reqs], (long long)p->total_ctx,
                  (long long)p->total_blk);
  }
  return ok();
}

size_t dflash_block_attention_workspace_size(const dflash_block_attn_params* p) {
  if (dflash_block_attention_check(p) != DFLASH_OK) return 0;
  dflash::AttnPlan plan;
  dflash::plan_block_attention(*p, kPlanComputeUnits, false, &plan);
  return plan.bytes;
}

size_t dflash_block_attention_paged_workspace_size(const dflash_block_attn_params* p) {
  if (dflash_block_attention_check(p) != DFLASH_OK) return 0;
  if (p->split_keys > kPagedMaxUnitKeys) return 0;
  dflash::AttnPlan plan;
  dflash::plan_block_attention(*p, kPlanComputeUnits, true, &plan);
  return plan.bytes;
}

}  // extern "C"

namespace {

// Shared by the packed and the paged entry points (pg == NULL: packed).
dflash_status block_attention_impl(const char* who, const dflash_block_attn_params* p,
                                   const dflash_paged_ctx* pg, const dflash_qk_prologue* prologue,
                                   const int32_t* cu_ctx_lens, const int32_t* cu_blk_lens,
                                   const void* q, const void* k_blk, const void* v_blk,
                                   const void* k_ctx, const void* v_ctx, void* out,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  dflash_status st = dflash_block_attention_check(p);
  if (st != DFLASH_OK) return st;
  if (pg) {
    if (pg->page_size != 16)
      return fail(DFLASH_ERR_UNSUPPORTED, "%s: page_size must be 16 (got %d)", who, pg->page_size);
    if (pg->max_pages_per_req < 1 || pg->num_pages < 1)
      return fail(DFLASH_ERR_INVALID_ARG, "%s: max_pages_per_req and num_pages must be >= 1", who);
    if (p->split_keys > kPagedMaxUnitKeys)
      return fail(DFLASH_ERR_INVALID_ARG, "%s: split_keys must be <= %d over a paged store", who,
                  kPagedMaxUnitKeys);
    if (p->total_blk > 0 && p->total_ctx > 0 && (!pg->block_table || !aligned(pg->block_table, 4)))
      return fail(DFLASH_ERR_INVALID_ARG, "%s: block_table is NULL or misaligned", who);
  }
  if (p->total_blk == 0) return ok();
  if (!cu_ctx_lens || !cu_blk_lens)
    return fail(DFLASH_ERR_INVALID_ARG, "%s: cu_ctx_lens/cu_blk_lens are NULL", who);
  if (!q || !k_blk || !v_blk || !out)
    return fail(DFLASH_ERR_INVALID_ARG, "%s: q/k_blk/v_blk/out must not be NULL", who);
  if (p->total_ctx > 0 && (!k_ctx || !v_ctx))
    return fail(DFLASH_ERR_INVALID_ARG, "%s: context K/V are NULL but total_ctx > 0", who);
  const void* tens[] = {q, k_blk, v_blk, out, k_ctx, v_ctx};
  for (const void* t : tens)
    if (t && !aligned(t, 16))
      return fail(DFLASH_ERR_INVALID_ARG, "%s: tensors must be 16-byte aligned", who);
  dflash::AttnPlan plan;
  dflash::plan_block_attention(*p, kPlanComputeUnits, pg != nullptr, &plan);
  if (plan.bytes > 0) {
    if (!workspace)
      return fail(DFLASH_ERR_WORKSPACE, "%s: workspace is NULL (%zu bytes needed)", who, plan.bytes);
    if (!aligned(workspace, 256))
      return fail(DFLASH_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", who);
    if (workspace_bytes < plan.bytes)
      return fail(DFLASH_ERR_WORKSPACE, "%s: workspace has %zu bytes, %zu needed", who,
                  workspace_bytes, plan.bytes);
  }
  if (prologue) {
    if (p->dtype != DFLASH_BF16)
      return fail(DFLASH_ERR_UNSUPPORTED, "%s: the fused prologue needs bf16", who);
    if (p->max_blk_len > 64)
      return fail(DFLASH_ERR_UNSUPPORTED, "%s: the fused prologue needs max_blk_len <= 64 (got %d)",
                  who, p->max_blk_len);
    if (!prologue->q_norm_w || !prologue->k_norm_w || !prologue->positions || !prologue->rope_table)
      return fail(DFLASH_ERR_INVALID_ARG, "%s: NULL pointer in the prologue", who);
    if (!aligned(prologue->q_norm_w, 16) || !aligned(prologue->k_norm_w, 16) ||
        !aligned(prologue->rope_table, 16))
      return fail(DFLASH_ERR_INVALID_ARG, "%s: prologue tensors must be 16-byte aligned", who);
    if (prologue->max_pos < 1)
      return fail(DFLASH_ERR_INVALID_ARG, "%s: prologue max_pos must be >= 1", who);
    if (!(prologue->eps >= 0.f) || !std::isfinite(prologue->eps))
      return fail(DFLASH_ERR_INVALID_ARG, "%s: prologue eps must be finite and >= 0", who);
  }
  if (plan.units * p->num_kv_heads > INT32_MAX)
    return fail(DFLASH_ERR_UNSUPPORTED, "%s: too many work units", who);
  if (validate_enabled()) {
    std::vector<int32_t> cc, cb;
    st = fetch_i32(who, "cu_ctx_lens", cu_ctx_lens, (int64_t)p->num_reqs + 1, &cc, stream);
    if (st == DFLASH_OK) st = fetch_i32(who, "cu_blk_lens", cu_blk_lens, (int64_t)p->num_reqs + 1, &cb, stream);
    if (st == DFLASH_OK) st = check_cu(who, "cu_ctx_lens", cc, p->total_ctx, -1, p->host_cu_ctx_lens);
    if (st == DFLASH_OK)
      st = check_cu(who, "cu_blk_lens", cb, p->total_blk, p->max_blk_len, p->host_cu_blk_lens);
    if (st == DFLASH_OK && prologue)
      st = check_positions(who, prologue->positions, p->total_blk, prologue->max_pos, stream);
    if (st == DFLASH_OK && pg && p->total_ctx > 0) {
      std::vector<int32_t> bt;
      st = fetch_i32(who, "block_table", pg->block_table,
                     (int64_t)p->num_reqs * pg->max_pages_per_req, &bt, stream);
      for (int32_t r = 0; st == DFLASH_OK && r < p->num_reqs; ++r) {
        const int64_t pages = ((int64_t)cc[r + 1] - cc[r] + pg->page_size - 1) / pg->page_size;
        if (pages > pg->max_pages_per_req)
          st = fail(DFLASH_ERR_INVALID_ARG, "%s: request %d needs %lld pages, more than max_pages_per_req %d",
                    who, r, (long long)pages, pg->max_pages_per_req);
        for (int64_t i = 0; st == DFLASH_OK && i < pages; ++i) {
          const int32_t id = bt[(size_t)((int64_t)r * pg->max_pages_per_req + i)];
          if (id < 0 || id >= pg->num_pages)
            st = fail(DFLASH_ERR_INVALID_ARG, "%s: block_table[%d][%lld] = %d is outside [0, %lld)", who,
                      r, (long long)i, id, (long long)pg->num_pages);
        }
      }
    }
    if (st != DFLASH_OK) return st;
  }
  return hip_status(dflash::launch_block_attention(*p, plan, prologue, pg, cu_ctx_lens, cu_blk_lens,
                                                   q, k_blk, v_blk, k_ctx, v_ctx, out, workspace,
                                                   (hipStream_t)stream),
                    "block_attention launch");
}

}  // namespace

extern "C" {

dflash_status dflash_block_attention(const dflash_block_attn_params* p,
                                     const dflash_qk_prologue* prologue, const int32_t* cu_ctx_lens,
                                     const int32_t* cu_blk_lens, const void* q, const void* k_blk,
                                     const void* v_blk, const void* k_ctx, const void* v_ctx,
                                     void* out, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  return block_attention_impl("block_attention", p, nullptr, prologue, cu_ctx_lens, cu_blk_lens, q,
                              k_blk, v_blk, k_ctx, v_ctx, out, workspace, workspace_bytes, stream);
}

dflash_status dflash_block_attention_noalloc(const dflash_block_attn_params* p,
                                             const dflash_qk_prologue* prologue,
                                             const int32_t* cu_ctx_lens,
                                             const int32_t* cu_blk_lens, const void* q,
                                             const void* k_blk, const void* v_blk,
                                             const void* k_ctx, const void* v_ctx, void* out,
                                             void* stream) {
  dflash_status st = dflash_block_attention_check(p);
  if (st != DFLASH_OK) return st;
  dflash::AttnPlan plan;
  dflash::plan_block_attention(*p, kPlanComputeUnits, false, &plan);
  if (plan.bytes > DFLASH_NOALLOC_SCRATCH_BYTES)
    return fail(DFLASH_ERR_WORKSPACE,
                "block_attention_noalloc: this batch needs %zu bytes of scratch, more than the "
                "%zu the library holds per GPU (call dflash_block_attention with a workspace)",
                plan.bytes, (size_t)DFLASH_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (plan.bytes > 0 && p->total_blk > 0) {
    const hipError_t e = dflash::noalloc_scratch(&ws);
    if (e != hipSuccess) return hip_status(e, "block_attention_noalloc: scratch address");
  }
  return block_attention_impl("block_attention_noalloc", p, nullptr, prologue, cu_ctx_lens,
                              cu_blk_lens, q, k_blk, v_blk, k_ctx, v_ctx, out, ws,
                              DFLASH_NOALLOC_SCRATCH_BYTES, stream);
}

dflash_status dflash_block_attention_paged(const dflash_block_attn_params* p,
                                           const dflash_paged_ctx* pg,
                                           const dflash_qk_prologue* prologue,
                                           const int32_t* cu_ctx_lens,
                                           const int32_t* cu_blk_lens, const void* q,
                                           const void* k_blk, const void* v_blk,
                                           const void* k_pool, const void* v_pool, void* out,
                                           void* workspace, size_t workspace_bytes,
                                           void* stream) {
  if (!pg) return fail(DFLASH_ERR_INVALID_ARG, "block_attention_paged: pg is NULL");
  return block_attention_impl("block_attention_paged", p, pg, prologue, cu_ctx_lens, cu_blk_lens,
                              q, k_blk, v_blk, k_pool, v_pool, out, workspace, workspace_bytes,
                              stream);
}

dflash_status dflash_kv_scatter(dflash_dtype dtype, const void* k_src, const void* v_src,
                                const int32_t* slot_mapping, int64_t T, int32_t num_kv_heads,
                                int32_t head_dim, void* k_pool, void* v_pool, int64_t num_slots,
                                void* stream) {
  if (dtype != DFLASH_F32 && dtype != DFLASH_BF16)
    return fail(DFLASH_ERR_INVALID_ARG, "kv_scatter: unknown dtype %d", (int)dtype);
  if (T < 0 || num_slots < 0 || num_kv_heads < 1 || head_dim < 1)
    return fail(DFLASH_ERR_INVALID_ARG, "kv_scatter: sizes must be non-negative (heads >= 1)");
  const int64_t row_bytes = (int64_t)num_kv_heads * head_dim * (dtype == DFLASH_BF16 ? 2 : 4);
  if (row_bytes % 16 != 0)
    return fail(DFLASH_ERR_UNSUPPORTED, "kv_scatter: a row must be a multiple of 16 bytes");
  if (T == 0 || num_slots == 0) return ok();
  if (!k_src || !v_src || !slot_mapping || !k_pool || !v_pool)
    return fail(DFLASH_ERR_INVALID_ARG, "kv_scatter: NULL pointer argument");
  if (!aligned(k_src, 16) || !aligned(v_src, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16))
    return fail(DFLASH_ERR_INVALID_ARG, "kv_scatter: tensors must be 16-byte aligned");
  if (T > ((int64_t)1 << 40) || num_slots > ((int64_t)1 << 40))
    return fail(DFLASH_ERR_INVALID_ARG, "kv_scatter: too many rows");
  if (validate_enabled()) {
    std::vector<int32_t> slots;
    const dflash_status st = fetch_i32("kv_scatter", "slot_mapping", slot_mapping, T, &slots, stream);
    if (st != DFLASH_OK) return st;
    std::vector<int32_t> in_range;
    for (int32_t v : slots)
      if (v >= 0 && v < num_slots) in_range.push_back(v);
    std::sort(in_range.begin(), in_range.end());
    const auto dup = std::adjacent_find(in_range.begin(), in_range.end());
    if (dup != in_range.end())
      return fail(DFLASH_ERR_INVALID_ARG, "kv_scatter: slot %d is written by more than one row", *dup);
  }
  return hip_status(dflash::launch_kv_scatter(dtype, k_src, v_src, slot_mapping, T, num_kv_heads,
                                              head_dim, k_pool, v_pool, num_slots,
                                              (hipStream_t)stream),
                    "kv_scatter launch");
}

// Calls with fewer rows than one tile of the large-row kernel (a propose
// step appending its verified rows) take the projection-GEMM path.
constexpr int64_t kCtxKvRowsPath = 256;
// Upper bound on the context projection's output width (Hkv * Dh) and on its
// hidden size: keeps every product of the two in the planners inside 32 bits.
constexpr int32_t kMaxProjDim = 1 << 20;

size_t dflash_context_kv_workspace_size(int64_t T, int32_t hidden_size, int32_t num_kv_heads,
                                        int32_t head_dim) {
  if (T < 0 || hidden_size < 1 || num_kv_heads < 1 || head_dim < 1) return 0;
  // sizes the call itself rejects (and whose products would not fit 32 bits)
  if ((int64_t)num_kv_heads * head_dim > kMaxProjDim || hidden_size > kMaxProjDim) return 0;
  if (T < kCtxKvRowsPath)
    return dflash::context_kv_rows_workspace_bytes(T, hidden_size, num_kv_heads, head_dim,
                                                   kPlanComputeUnits);
  return dflash::context_kv_workspace_bytes(T, hidden_size, num_kv_heads, head_dim);
}

dflash_status dflash_context_kv(const void* hidden, const float* hidden_norm_w, const void* w_k,
                                const void* w_v, const float* k_norm_w, const int32_t* positions,
                                int64_t T, int32_t hidden_size, int32_t num_kv_heads,
                                int32_t head_dim, float eps, const float* rope_table,
                                int32_t max_pos, void* k_out, void* v_out, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (T < 0) return fail(DFLASH_ERR_INVALID_ARG, "context_kv: T must be >= 0");
  if (num_kv_heads < 1) return fail(DFLASH_ERR_INVALID_ARG, "context_kv: num_kv_heads must be >= 1");
  if (head_dim != 128)
    return fail(DFLASH_ERR_UNSUPPORTED, "context_kv: head_dim %d is not supported (128)", head_dim);
  if ((int64_t)num_kv_heads * head_dim > kMaxProjDim)
    return fail(DFLASH_ERR_INVALID_ARG, "context_kv: num_kv_heads * head_dim must be <= %d", kMaxProjDim);
  if (hidden_size < 64 || hidden_size % 64 != 0 || hidden_size > kMaxProjDim)
    return fail(DFLASH_ERR_UNSUPPORTED, "context_kv: hidden_size must be a multiple of 64 in [64, %d]",
                kMaxProjDim);
  if ((num_kv_heads * head_dim) % 256 != 0)
    return fail(DFLASH_ERR_UNSUPPORTED, "context_kv: num_kv_heads * head_dim must be a multiple of 256");
  if (!(eps >= 0.f) || !std::isfinite(eps))
    return fail(DFLASH_ERR_INVALID_ARG, "context_kv: eps must be finite and >= 0");
  if (max_pos < 1) return fail(DFLASH_ERR_INVALID_ARG, "context_kv: max_pos must be >= 1");
  if (T == 0) return ok();
  const void* ptrs[] = {hidden, hidden_norm_w, w_k, w_v, k_norm_w, positions, rope_table, k_out, v_out};
  for (const void* t : ptrs)
    if (!t) return fail(DFLASH_ERR_INVALID_ARG, "context_kv: NULL pointer argument");
  const void* al[] = {hidden, hidden_norm_w, w_k, w_v, k_norm_w, rope_table, k_out, v_out};
  for (const void* t : al)
    if (!aligned(t, 16)) return fail(DFLASH_ERR_INVALID_ARG, "context_kv: tensors must be 16-byte aligned");
  const size_t need = dflash_context_kv_workspace_size(T, hidden_size, num_kv_heads, head_dim);
  if (need > 0) {
    if (!workspace) return fail(DFLASH_ERR_WORKSPACE, "context_kv: workspace is NULL (%zu bytes needed)", need);
    if (!aligned(workspace, 256))
      return fail(DFLASH_ERR_WORKSPACE, "context_kv: workspace must be 256-byte aligned");
    if (workspace_bytes < need)
      return fail(DFLASH_ERR_WORKSPACE, "context_kv: workspace has %zu bytes, %zu needed",
                  workspace_bytes, need);
  }
  if (T < kCtxKvRowsPath && hidden_size > 8192)
    return fail(DFLASH_ERR_UNSUPPORTED, "context_kv: calls of fewer than %lld rows need hidden_size <= 8192",
                (long long)kCtxKvRowsPath);
  if (validate_enabled()) {
    const dflash_status st = check_positions("context_kv", positions, T, max_pos, stream);
    if (st != DFLASH_OK) return st;
  }
  if (T < kCtxKvRowsPath)
    return hip_status(dflash::launch_context_kv_rows(hidden, hidden_norm_w, w_k, w_v, k_norm_w,
                                                     positions, T, hidden_size, num_kv_heads,
                                                     head_dim, eps, rope_table, max_pos, k_out,
                                                     v_out, workspace, kPlanComputeUnits,
                                                     (hipStream_t)stream),
                      "context_kv launch");
  return hip_status(dflash::launch_context_kv(hidden, hidden_norm_w, w_k, w_v, k_norm_w, positions,
                                              T, hidden_size, num_kv_heads, head_dim, eps,
                                              rope_table, max_pos, k_out, v_out, workspace,
                                              (hipStream_t)stream),
                    "context_kv launch");
}

size_t dflash_block_qkv_workspace_size(int64_t T, int32_t hidden_size, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim) {
  if (T < 0 || T > INT32_MAX || hidden_size < 64 || num_q_heads < 1 || num_kv_heads < 1 || head_dim < 1)
    return 0;
  if (((int64_t)num_q_heads + 2 * (int64_t)num_kv_heads) * head_dim > INT32_MAX / 2 ||
      hidden_size > kMaxProjDim)
    return 0;  // rejected by the call
  return dflash::block_qkv_workspace_bytes(T, hidden_size, num_q_heads, num_kv_heads, head_dim,
                                           kPlanComputeUnits);
}

dflash_status dflash_block_qkv(const void* hidden, void* residual, const float* norm_w,
                               const void* w_qkv, int64_t T, int32_t hidden_size,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               float eps, void* q, void* k, void* v, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (T < 0 || T > INT32_MAX) return fail(DFLASH_ERR_INVALID_ARG, "block_qkv: T must be in [0, 2^31)");
  if (num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads != 0)
    return fail(DFLASH_ERR_INVALID_ARG, "block_qkv: need Hq >= 1, Hkv >= 1 and Hq %% Hkv == 0");
  if (head_dim != 64 && head_dim != 128)
    return fail(DFLASH_ERR_UNSUPPORTED, "block_qkv: head_dim %d is not supported (64 or 128)", head_dim);
  if (hidden_size < 64 || hidden_size % 64 != 0 || hidden_size > 8192)
    return fail(DFLASH_ERR_UNSUPPORTED, "block_qkv: hidden_size must be a multiple of 64 in [64, 8192]");
  if (((int64_t)num_q_heads + 2 * (int64_t)num_kv_heads) * head_dim > INT32_MAX / 2)
    return fail(DFLASH_ERR_INVALID_ARG, "block_qkv: too many heads");
  if (!(eps >= 0.f) || !std::isfinite(eps))
    return fail(DFLASH_ERR_INVALID_ARG, "block_qkv: eps must be finite and >= 0");
  if (T == 0) return ok();
  const void* ptrs[] = {hidden, norm_w, w_qkv, q, k, v};
  for (const void* t : ptrs)
    if (!t) return fail(DFLASH_ERR_INVALID_ARG, "block_qkv: NULL pointer argument");
  const void* al[] = {hidden, norm_w, w_qkv, q, k, v, residual};
  for (const void* t : al)
    if (t && !aligned(t, 16)) return fail(DFLASH_ERR_INVALID_ARG, "block_qkv: tensors must be 16-byte aligned");
  const size_t need = dflash::block_qkv_workspace_bytes(T, hidden_size, num_q_heads, num_kv_heads,
                                                        head_dim, kPlanComputeUnits);
  if (!workspace) return fail(DFLASH_ERR_WORKSPACE, "block_qkv: workspace is NULL (%zu bytes needed)", need);
  if (!aligned(workspace, 256)) return fail(DFLASH_ERR_WORKSPACE, "block_qkv: workspace must be 256-byte aligned");
  if (workspace_bytes < need)
    return fail(DFLASH_ERR_WORKSPACE, "block_qkv: workspace has %zu bytes, %zu needed", workspace_bytes, need);
  return hip_status(dflash::launch_block_qkv(hidden, residual, norm_w, w_qkv, T, hidden_size,
                                             num_q_heads, num_kv_heads, head_dim, eps, q, k, v,
                                             workspace, kPlanComputeUnits, (hipStream_t)stream),
                    "block_qkv launch");
}

size_t dflash_o_proj_workspace_size(int64_t T, int32_t hidden_size, int32_t in_dim) {
  if (T < 0 || T > INT32_MAX || hidden_size < 64 || in_dim < 64) return 0;
  return dflash::o_proj_workspace_bytes(T, hidden_size, in_dim, kPlanComputeUnits);
}

dflash_status dflash_o_proj(const void* attn, const void* w_o, int64_t T, int32_t hidden_size,
                            int32_t in_dim, void* out, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (T < 0 || T > INT32_MAX) return fail(DFLASH_ERR_INVALID_ARG, "o_proj: T must be in [0, 2^31)");
  if (hidden_size < 64 || hidden_size % 64 != 0)
    return fail(DFLASH_ERR_UNSUPPORTED, "o_proj: hidden_size must be a positive multiple of 64");
  if (in_dim < 64 || in_dim % 64 != 0)
    return fail(DFLASH_ERR_UNSUPPORTED, "o_proj: in_dim must be a positive multiple of 64");
  if (T == 0) return ok();
  if (!attn || !w_o || !out) return fail(DFLASH_ERR_INVALID_ARG, "o_proj: NULL pointer argument");
  if (!aligned(attn, 16) || !aligned(w_o, 16) || !aligned(out, 16))
    return fail(DFLASH_ERR_INVALID_ARG, "o_proj: tensors must be 16-byte aligned");
  const size_t need = dflash::o_proj_workspace_bytes(T, hidden_size, in_dim, kPlanComputeUnits);
  if (need > 0) {
    if (!workspace) return fail(DFLASH_ERR_WORKSPACE, "o_proj: workspace is NULL (%zu bytes needed)", need);
    if (!aligned(workspace, 256)) return fail(DFLASH_ERR_WORKSPACE, "o_proj: workspace must be 256-byte aligned");
    if (workspace_bytes < need)
      return fail(DFLASH_ERR_WORKSPACE, "o_proj: workspace has %zu bytes, %zu needed", workspace_bytes, need);
  }
  return hip_status(dflash::launch_o_proj(attn, w_o, T, hidden_size, in_dim, out, workspace,
                                          kPlanComputeUnits, (hipStream_t)stream),
                    "o_proj launch");
}

dflash_status dflash_prepare_inputs(const dflash_prepare_params* p,
                                    const dflash_prepare_inputs_in* in,
                                    const dflash_prepare_inputs_out* out, void* stream) {
  if (!p || !in || !out) return fail(DFLASH_ERR_INVALID_ARG, "prepare_inputs: NULL argument");
  if (p->num_reqs < 1) return fail(DFLASH_ERR_INVALID_ARG, "prepare_inputs: num_reqs must be >= 1");
  if (p->max_num_reqs < p->num_reqs)
    return fail(DFLASH_ERR_INVALID_ARG, "prepare_inputs: max_num_reqs < num_reqs");
  if (p->num_query_per_req < 1)
    return fail(DFLASH_ERR_INVALID_ARG, "prepare_inputs: num_query_per_req must be >= 1");
  if ((int64_t)p->max_num_tokens < (int64_t)p->num_reqs * p->num_query_per_req)
    return fail(DFLASH_ERR_INVALID_ARG, "prepare_inputs: max_num_tokens < num_reqs * num_query_per_req");
  if (p->num_speculative_steps != p->num_query_per_req - (p->sample_from_anchor ? 0 : 1))
    return fail(DFLASH_ERR_INVALID_ARG,
                "prepare_inputs: num_speculative_steps must be num_query_per_req - %d",
                p->sample_from_anchor ? 0 : 1);
  if (p->block_size < 1 || p->block_table_stride < 1 || p->max_model_len < 1 || p->num_states < 1)
    return fail(DFLASH_ERR_INVALID_ARG,
                "prepare_inputs: block_size, block_table_stride, max_model_len and num_states must be >= 1");
  if (p->num_target_tokens < 1)
    return fail(DFLASH_ERR_INVALID_ARG, "prepare_inputs: num_target_tokens must be >= 1");
  const void* ins[] = {in->idx_mapping, in->target_query_start_loc, in->target_positions,
                       in->num_rejected, in->num_sampled, in->last_sampled,
                       in->next_prefill_tokens, in->block_table};
  for (const void* t : ins)
    if (!t) return fail(DFLASH_ERR_INVALID_ARG, "prepare_inputs: NULL input array");
  const void* outs[] = {out->input_ids, out->query_positions, out->query_start_loc, out->seq_lens,
                        out->query_slot_mapping, out->context_positions,
                        out->context_slot_mapping, out->sample_indices, out->sample_pos,
                        out->sample_idx_mapping, out->ctx_cu};
  for (const void* t : outs)
    if (!t) return fail(DFLASH_ERR_INVALID_ARG, "prepare_inputs: NULL output array");
  return hip_status(dflash::launch_prepare_inputs(*p, *in, *out, (hipStream_t)stream),
                    "prepare_inputs launch");
}

size_t dflash_fc_combine_workspace_size(int64_t T, int32_t hidden_size, int32_t num_taps) {
  if (T < 0 || T > INT32_MAX || hidden_size < 64 || num_taps < 1) return 0;
  if ((int64_t)hidden_size * num_taps > INT32_MAX / 2) return 0;  // rejected by the call
  return dflash::fc_combine_workspace_bytes(T, hidden_size, num_taps, kPlanComputeUnits);
}

dflash_status dflash_fc_combine(const float* aux, const void* w_fc, int64_t T, int32_t hidden_size,
                                int32_t num_taps, void* out, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (T < 0 || T > INT32_MAX) return fail(DFLASH_ERR_INVALID_ARG, "fc_combine: T must be in [0, 2^31)");
  if (hidden_size < 64 || hidden_size % 64 != 0)
    return fail(DFLASH_ERR_UNSUPPORTED, "fc_combine: hidden_size must be a positive multiple of 64");
  if (num_taps < 1 || (int64_t)hidden_size * num_taps > INT32_MAX / 2)
    return fail(DFLASH_ERR_INVALID_ARG, "fc_combine: num_taps must be >= 1 (and H * taps < 2^30)");
  if (T == 0) return ok();
  if (!aux || !w_fc || !out) return fail(DFLASH_ERR_INVALID_ARG, "fc_combine: NULL pointer argument");
  if (!aligned(aux, 16) || !aligned(w_fc, 16) || !aligned(out, 16))
    return fail(DFLASH_ERR_INVALID_ARG, "fc_combine: tensors must be 16-byte aligned");
  const size_t need = dflash::fc_combine_workspace_bytes(T, hidden_size, num_taps, kPlanComputeUnits);
  if (!workspace) return fail(DFLASH_ERR_WORKSPACE, "fc_combine: workspace is NULL (%zu bytes needed)", need);
  if (!aligned(workspace, 256)) return fail(DFLASH_ERR_WORKSPACE, "fc_combine: workspace must be 256-byte aligned");
  if (workspace_bytes < need)
    return fail(DFLASH_ERR_WORKSPACE, "fc_combine: workspace has %zu bytes, %zu needed", workspace_bytes, need);
  return hip_status(dflash::launch_fc_combine(aux, w_fc, T, hidden_size, num_taps, out, workspace,
                                              kPlanComputeUnits, (hipStream_t)stream),
                    "fc_combine launch");
}

}  // extern "C"
