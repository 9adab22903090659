// Appending rows to the paged context store: an index copy of K and V rows
// to flat pool slots ("qwen3_dflash.cpp" page, the paged draft-KV store:
// appended context rows are scattered to their slots, slot = page *
// page_size + offset). HBM-bound: each row is read once and written once.
#include "dflash_device.h"
#include "dflash_internal.h"

namespace dflash {
namespace {

// One thread per 16-byte chunk of a row (K and V); rows whose slot is outside
// [0, num_slots) are skipped (the padding slot -1 among them).
__global__ __launch_bounds__(256) void kv_scatter_kernel(const uint4* __restrict__ ks,
                                                         const uint4* __restrict__ vs,
                                                         const int32_t* __restrict__ slots,
                                                         int64_t rows, int64_t chunks_per_row,
                                                         uint4* __restrict__ kp,
                                                         uint4* __restrict__ vp, int64_t num_slots) {
  // every argument in one batch of scalar loads (no dependent argument reads)
  asm volatile("" ::"s"(ks), "s"(vs), "s"(slots), "s"(rows), "s"(chunks_per_row), "s"(kp), "s"(vp),
               "s"(num_slots));
  const int64_t total = rows * chunks_per_row;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / chunks_per_row;
    const int64_t c = i - t * chunks_per_row;
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= num_slots) continue;
    kp[slot * chunks_per_row + c] = ks[i];
    vp[slot * chunks_per_row + c] = vs[i];
  }
}

}  // namespace

hipError_t launch_kv_scatter(dflash_dtype dt, const void* k_src, const void* v_src,
                             const int32_t* slots, int64_t rows, int32_t hkv, int32_t dh,
                             void* k_pool, void* v_pool, int64_t num_slots, hipStream_t s) {
  const int64_t row_bytes = (int64_t)hkv * dh * (dt == DFLASH_BF16 ? 2 : 4);
  const int64_t cpr = row_bytes / 16;
  const int64_t total = rows * cpr;
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 256 * 64);
  hipLaunchKernelGGL(kv_scatter_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     (const uint4*)k_src, (const uint4*)v_src, slots, rows, cpr, (uint4*)k_pool,
                     (uint4*)v_pool, num_slots);
  return hipGetLastError();
}

}  // namespace dflash
