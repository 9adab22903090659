// Host-side interface between the C-ABI layer and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dflash.h"

namespace dflash {

// A one-dimensional grid larger than a launch can address is refused
// (hipErrorInvalidConfiguration) rather than truncated to 32 bits.
inline bool grid_fits(int64_t blocks) { return blocks >= 0 && blocks <= 0x7fffffff; }

hipError_t launch_rope_table(float* table, int32_t max_pos, int32_t head_dim, double theta,
                             hipStream_t s);

hipError_t launch_qk_norm_rope(dflash_dtype dt, void* q, void* k, const float* wq,
                               const float* wk, const int32_t* pos, int64_t rows, int32_t hq,
                               int32_t hkv, int32_t dh, float eps, const float* table,
                               int32_t max_pos, hipStream_t s);

// Work decomposition of one block-attention call (host side, no device access).
struct AttnPlan {
  int32_t group;      // Hq / Hkv
  int32_t qtiles;     // bound on 64-row query tiles per (request, kv-head)
  int32_t chunk;      // keys per work unit (multiple of 64)
  int64_t units;      // bound on work units per kv-head (grid = units * Hkv)
  int64_t units_pref; // unit budget the split is chosen for first (<= units)
  size_t off_counters, off_part_o, off_part_ml, bytes;
  size_t off_trace;    // phase-trace records (diagnostic build only; else == bytes)
  int64_t trace_main;  // records of the main kernel's workgroups (diagnostic build)
  int32_t cus;         // compute units the plan was made for
};
bool plan_block_attention(const dflash_block_attn_params& p, int num_cus, bool paged,
                          AttnPlan* plan);

hipError_t launch_block_attention(const dflash_block_attn_params& p, const AttnPlan& plan,
                                  const dflash_qk_prologue* pro, const dflash_paged_ctx* pg,
                                  const int32_t* cu_ctx, const int32_t* cu_blk, const void* q,
                                  const void* kb, const void* vb, const void* kc, const void* vc,
                                  void* out, void* ws, hipStream_t s);

hipError_t launch_kv_scatter(dflash_dtype dt, const void* k_src, const void* v_src,
                             const int32_t* slots, int64_t rows, int32_t hkv, int32_t dh,
                             void* k_pool, void* v_pool, int64_t num_slots, hipStream_t s);

size_t context_kv_workspace_bytes(int64_t rows, int32_t hidden, int32_t hkv, int32_t dh);
hipError_t launch_context_kv(const void* hidden, const float* hnw, const void* wk,
                             const void* wv, const float* knw, const int32_t* pos, int64_t rows,
                             int32_t hidden_size, int32_t hkv, int32_t dh, float eps,
                             const float* table, int32_t max_pos, void* k_out, void* v_out,
                             void* ws, hipStream_t s);

size_t block_qkv_workspace_bytes(int64_t T, int32_t hidden, int32_t hq, int32_t hkv, int32_t dh,
                                 int num_cus);
hipError_t launch_block_qkv(const void* hidden, void* residual, const float* norm_w,
                            const void* w_qkv, int64_t T, int32_t hidden_size, int32_t hq,
                            int32_t hkv, int32_t dh, float eps, void* q, void* k, void* v,
                            void* ws, int num_cus, hipStream_t s);
size_t o_proj_workspace_bytes(int64_t T, int32_t hidden, int32_t in_dim, int num_cus);
hipError_t launch_o_proj(const void* attn, const void* w_o, int64_t T, int32_t hidden,
                         int32_t in_dim, void* out, void* ws, int num_cus, hipStream_t s);

size_t context_kv_rows_workspace_bytes(int64_t T, int32_t hidden, int32_t hkv, int32_t dh,
                                       int num_cus);
hipError_t launch_context_kv_rows(const void* hidden, const float* hnw, const void* wk,
                                  const void* wv, const float* knw, const int32_t* pos, int64_t T,
                                  int32_t hidden_size, int32_t hkv, int32_t dh, float eps,
                                  const float* table, int32_t max_pos, void* k_out, void* v_out,
                                  void* ws, int num_cus, hipStream_t s);
size_t fc_combine_workspace_bytes(int64_t T, int32_t hidden, int32_t taps, int num_cus);
hipError_t launch_fc_combine(const float* aux, const void* w_fc, int64_t T, int32_t hidden,
                             int32_t taps, void* out, void* ws, int num_cus, hipStream_t s);

// Device address of the current device's copy of the allocation-free entry
// point's scratch array (DFLASH_NOALLOC_SCRATCH_BYTES bytes), looked up on the
// first call on each device.
hipError_t noalloc_scratch(void** addr);

hipError_t launch_prepare_inputs(const dflash_prepare_params& p, const dflash_prepare_inputs_in& in,
                                 const dflash_prepare_inputs_out& out, hipStream_t s);

}  // namespace dflash
