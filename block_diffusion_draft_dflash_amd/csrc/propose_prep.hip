// Integer preparation of one DFlash propose step on the device.
//
// "qwen3_dflash.cpp" page, PrepareDflashInputs: per request, the step's
// verified target rows become context rows (positions and KV slots), the last
// num_rejected of them are rolled back, and the block of 1 + k rows -- the
// anchor token (the token last sampled, or the next prefill token when the
// request sampled nothing) followed by mask tokens -- starts right after the
// last kept position; slots come from the request's block table (page =
// position / block_size clamped to the last page). The sample maps pick the
// block rows to sample, and the tail of every padded array is filled so that
// a captured graph replays over a smaller batch safely. Integer only: the
// kernel's outputs are exactly the host loop's.
#include <algorithm>

#include "dflash_device.h"
#include "dflash_internal.h"

namespace dflash {
namespace {

constexpr int PT = 256;

__device__ __forceinline__ int64_t clamp64(int64_t x, int64_t lo, int64_t hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

// The last kept position of request r (index clamped into the target rows).
__device__ __forceinline__ int64_t last_kept_pos(const dflash_prepare_params& p,
                                                 const dflash_prepare_inputs_in& in, int32_t r) {
  const int64_t ntgt = p.num_target_tokens;
  const int64_t start = clamp64(in.target_query_start_loc[r], 0, ntgt);
  const int64_t end = clamp64(in.target_query_start_loc[r + 1], start, ntgt);
  const int64_t kept_end = end - in.num_rejected[r];
  return in.target_positions[clamp64(kept_end - 1, 0, ntgt - 1)];
}

// Workgroup r < num_reqs: request r. Workgroup num_reqs: the cumulative
// kept-context lengths and the padded tails.
__global__ __launch_bounds__(PT) void prepare_inputs_kernel(dflash_prepare_params p,
                                                            dflash_prepare_inputs_in in,
                                                            dflash_prepare_inputs_out out) {
  const int32_t r = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t nqpr = p.num_query_per_req, nspec = p.num_speculative_steps;
  const int32_t R = p.num_reqs;
  if (r == R) {
    // Running sum of the kept-context lengths over the requests, PT requests
    // at a time: every thread loads its request's length (the loads of a
    // chunk are in flight together), then an inclusive scan across the
    // workgroup plus the carry of the chunks before. Unsigned arithmetic: the
    // same bits as the in-order two's-complement sum.
    __shared__ uint32_t wsum[PT / 64];
    uint32_t carry = 0;
    if (tid == 0) out.ctx_cu[0] = 0;
    for (int32_t base = 0; base < R; base += PT) {
      const int32_t i = base + tid;
      uint32_t x = i < R ? (uint32_t)(int32_t)(last_kept_pos(p, in, i) + 1) : 0u;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = __shfl_up(x, d, 64);
        if ((tid & 63) >= d) x += y;
      }
      if ((tid & 63) == 63) wsum[tid >> 6] = x;
      __syncthreads();
      uint32_t before = carry, total = 0;
#pragma unroll
      for (int wv = 0; wv < PT / 64; ++wv) {
        before += wv < (tid >> 6) ? wsum[wv] : 0u;
        total += wsum[wv];
      }
      if (i < R) out.ctx_cu[i + 1] = (int32_t)(before + x);
      carry += total;
      __syncthreads();  // wsum is rewritten by the next chunk
    }
    for (int64_t i = (int64_t)R + 1 + tid; i <= p.max_num_reqs; i += PT) out.ctx_cu[i] = (int32_t)carry;
    for (int64_t i = R + tid; i <= p.max_num_reqs; i += PT) out.query_start_loc[i] = R * nqpr;
    for (int64_t i = R + tid; i < p.max_num_reqs; i += PT) out.seq_lens[i] = 0;
    for (int64_t i = (int64_t)R * nspec + tid; i < (int64_t)p.max_num_reqs * nspec; i += PT) {
      out.sample_indices[i] = 0;
      out.sample_pos[i] = 0;
      out.sample_idx_mapping[i] = -1;
    }
    for (int64_t i = (int64_t)R * nqpr + tid; i < p.max_num_tokens; i += PT)
      out.query_slot_mapping[i] = -1;
    return;
  }
  // Device metadata is trusted but every index derived from it is clamped
  // into its buffer.
  const int64_t ntgt = p.num_target_tokens;
  const int32_t state = (int32_t)clamp64(in.idx_mapping[r], 0, p.num_states - 1);
  const int64_t start = clamp64(in.target_query_start_loc[r], 0, ntgt);
  const int64_t end = clamp64(in.target_query_start_loc[r + 1], start, ntgt);
  const int64_t last_kept = last_kept_pos(p, in, r);
  const int32_t anchor = in.num_sampled[r] > 0 ? in.last_sampled[state] : in.next_prefill_tokens[state];
  const int32_t* bt = in.block_table + (int64_t)r * p.block_table_stride;
  const int64_t bs = p.block_size;
  auto slot = [&](int64_t pos) -> int32_t {
    const int64_t page = clamp64(pos / bs, 0, p.block_table_stride - 1);
    return (int32_t)((int64_t)bt[page] * bs + pos % bs);
  };
  for (int64_t t = start + tid; t < end; t += PT) {
    const int64_t pos = in.target_positions[t];
    out.context_positions[t] = (int32_t)pos;
    out.context_slot_mapping[t] = slot(pos);
  }
  const int32_t first_sample = p.sample_from_anchor ? 0 : 1;
  for (int32_t off = tid; off < nqpr; off += PT) {
    const int64_t pos = last_kept + 1 + off;
    const int64_t qi = (int64_t)r * nqpr + off;
    out.input_ids[qi] = off == 0 ? anchor : p.mask_token_id;
    out.query_positions[qi] = (int32_t)std::min<int64_t>(pos, (int64_t)p.max_model_len - 1);
    out.query_slot_mapping[qi] = slot(pos);
    if (off >= first_sample) {
      const int64_t si = (int64_t)r * nspec + (off - first_sample);
      out.sample_indices[si] = (int32_t)qi;
      out.sample_pos[si] = (int32_t)(p.sample_from_anchor ? pos + 1 : pos);
      out.sample_idx_mapping[si] = state;
    }
  }
  if (tid == 0) {
    out.query_start_loc[r] = r * nqpr;
    out.seq_lens[r] = (int32_t)(last_kept + 1 + nqpr);
  }
}

}  // namespace

hipError_t launch_prepare_inputs(const dflash_prepare_params& p, const dflash_prepare_inputs_in& in,
                                 const dflash_prepare_inputs_out& out, hipStream_t s) {
  hipLaunchKernelGGL(prepare_inputs_kernel, dim3((unsigned)p.num_reqs + 1), dim3(PT), 0, s, p, in, out);
  return hipGetLastError();
}

}  // namespace dflash
