// Context K/V precompute: hidden RMSNorm -> K/V projection -> per-head k-norm
// -> NeoX RoPE on K; V raw.
//
// "qwen3_dflash.cpp" page, PrecomputeContextKVDevice: normed = RMSNorm(h,
// hidden_norm); K = normed W_k^T, V = normed W_v^T with W_k / W_v the K and V
// row slices of the merged qkv weight; per-head RMSNorm of K over head_dim with
// k_norm; RopeNeox on K at the context positions; bf16 storage (ContextKVDev).
//
// The row scale of the hidden RMSNorm factors out of the contraction:
//   K[t, o] = (1 / rms_t) * sum_j h[t, j] * (hidden_norm[j] * W_k[o, j]),
// so the weights are pre-multiplied by hidden_norm once per call (rounded to
// bf16, the reference rounds the normed activations instead) and 1/rms_t is
// applied in the GEMM epilogue. The GEMM (M = rows, N = 2 * Hkv * Dh, K = H)
// runs on v_mfma_f32_16x16x32_bf16 with 256x256 workgroup tiles; each wave owns
// 128 rows x one 128-wide head, so the k-norm and the rotate-half pairs
// (d, d + 64) are resolved in registers of one wave. The k-slices of A and B
// are copied HBM -> LDS directly (no register staging), NSTAGE - 1 slices
// ahead, with explicit waits and fence-free barriers.
#include <mutex>

#include "dflash_device.h"
#include "dflash_internal.h"

namespace dflash {
namespace {

constexpr int BM = 256, BN = 256, BK = 32, NT = 256;

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// W'[o, j] = bf16(W[o, j] * hidden_norm[j]) for the K rows then the V rows.
__global__ __launch_bounds__(256) void fold_weights_kernel(const bf16* __restrict__ wk,
                                                           const bf16* __restrict__ wv,
                                                           const float* __restrict__ hnw,
                                                           bf16* __restrict__ wout, int64_t kdim,
                                                           int32_t hidden) {
  const int64_t idx = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  const int64_t per = kdim * hidden;
  if (idx >= 2 * per) return;
  const bf16* src = idx < per ? wk + idx : wv + (idx - per);
  const int32_t col = (int32_t)(idx % hidden);
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(src);
  const float4 n0 = *reinterpret_cast<const float4*>(hnw + col);
  const float4 n1 = *reinterpret_cast<const float4*>(hnw + col + 4);
  const float n[8] = {n0.x, n0.y, n0.z, n0.w, n1.x, n1.y, n1.z, n1.w};
  bf16x8 o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = f2bf(bf2f(v[e]) * n[e]);
  *reinterpret_cast<bf16x8*>(wout + idx) = o;
}

// rstd[t] = 1 / sqrt(mean(h[t]^2) + eps); one wave per row.
__global__ __launch_bounds__(256) void row_rstd_kernel(const bf16* __restrict__ h,
                                                       float* __restrict__ rstd, int64_t rows,
                                                       int32_t hidden, float eps) {
  const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const bf16* p = h + row * hidden;
  float ss = 0.f;
  for (int32_t c = lane * 8; c < hidden; c += 512) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(p + c);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = bf2f(v[e]);
      ss += x * x;
    }
  }
  ss = group_sum<64>(ss);
  if (lane == 0) rstd[row] = 1.0f / sqrtf(ss / (float)hidden + eps);
}

struct CkvArgs {
  const bf16* h;        // [rows, H]
  const bf16* w;        // [N, H] folded weights, K rows then V rows
  const float* rstd;    // [rows]
  const float* knw;     // [Dh]
  const int32_t* pos;   // [rows]
  const float2* table;  // [max_pos][Dh/2]
  bf16* k_out;          // [rows, Hkv, Dh]
  bf16* v_out;
  int64_t rows;
  int32_t hidden, n, hkv, max_pos;
  float eps;
};

// A and B tiles are [256 rows][32 k] bf16 (64-byte rows, 4 chunks of 16 B);
// chunk c of row r is stored at c ^ ((r >> 2) & 3) so 16 consecutive rows read
// at one logical chunk touch distinct banks.
__device__ __forceinline__ int tswz(int row, int c) { return c ^ ((row >> 2) & 3); }

constexpr int NSTAGE = 4;  // LDS stages of (A, B) k-slices: NSTAGE - 1 in flight

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14; expcnt and lgkmcnt left at their no-wait maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Workgroup barrier without the memory fence of __syncthreads() (which would
// drain the k-slices still in flight).
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(NT) void ctx_kv_gemm_kernel(CkvArgs a) {
  constexpr int DH = 128;
  constexpr int HALF = DH / 2;
  constexpr int TILE = BM * BK;         // elements per A (or B) k-slice
  constexpr int CPW = TILE / 512 / 4;   // 1 KB copies per wave per operand per k-slice (4)
  constexpr int CPS = 2 * CPW;          // per thread per k-slice (A and B)
  extern __shared__ __attribute__((aligned(16))) bf16 smem[];  // [stage][A | B]

  // Block order: the dispatcher deals workgroups to the 8 XCDs round-robin.
  // Consecutive row blocks go to different XCDs and each XCD runs all column
  // tiles of its row blocks, so an XCD's L2 fetches each A row block once
  // (B, 16 MB at most, is shared through the last-level cache).
  const int ntn = a.n / BN;
  const int xcd = blockIdx.x % 8;
  const int slot = blockIdx.x / 8;
  const int64_t rb = (int64_t)(slot / ntn) * 8 + xcd;
  const int64_t row0 = rb * BM;
  if (row0 >= a.rows) return;
  const int col0 = (slot % ntn) * BN;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, m = lane & 15, j = lane >> 4;
  const int wm = w >> 1, wn = w & 1;

  // Copies: one wave-wide 16-byte-per-lane load fills 1 KB = 16 tile rows of
  // LDS in lane order; lane L takes the logical chunk the swizzle stores at
  // its slot. Rows past the end re-read the last row (their results are not
  // stored).
  const bf16* asrc[CPW];
  const bf16* bsrc[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int r = (w * CPW + i) * 16 + lane / 4;
    const int c = tswz(r, lane % 4);
    const int64_t grow = min(row0 + r, a.rows - 1);
    asrc[i] = a.h + grow * a.hidden + c * 8;
    bsrc[i] = a.w + (int64_t)(col0 + r) * a.hidden + c * 8;
  }
  auto dma = [](const bf16* src, bf16* dst) {
    const uint32_t lds_addr =
        __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(DF_LDS void*)dst);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds_addr), "v"(src)
                 : "memory", "m0");
  };
  auto issue = [&](int32_t ks) {
    bf16* as = smem + (ks % NSTAGE) * 2 * TILE;
    bf16* bs = as + TILE;
    const int32_t k0 = ks * BK;
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      dma(asrc[i] + k0, as + (w * CPW + i) * 512);
      dma(bsrc[i] + k0, bs + (w * CPW + i) * 512);
    }
  };

  f32x4 acc[8][8];
#pragma unroll
  for (int x = 0; x < 8; ++x)
#pragma unroll
    for (int y = 0; y < 8; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int32_t ksteps = a.hidden / BK;
#pragma unroll
  for (int t = 0; t < NSTAGE - 1; ++t)
    if (t < ksteps) issue(t);
  for (int32_t ks = 0; ks < ksteps; ++ks) {
    // own copies of slice ks landed (later slices may stay in flight); the
    // barrier publishes every wave's part and frees the stage of slice ks-1
    const int32_t after = min(ksteps - 1 - ks, NSTAGE - 2);
    if (after >= 2) wait_vmcnt<2 * CPS>();
    else if (after == 1) wait_vmcnt<CPS>();
    else wait_vmcnt<0>();
    block_barrier();
    if (ks + NSTAGE - 1 < ksteps) issue(ks + NSTAGE - 1);
    const bf16* as = smem + (ks % NSTAGE) * 2 * TILE;
    const bf16* bs = as + TILE;
    bf16x8 af[8], bfr[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const int ra = 128 * wm + 16 * x + m;
      af[x] = *reinterpret_cast<const bf16x8*>(as + ra * BK + tswz(ra, j) * 8);
      const int rb2 = 128 * wn + 16 * x + m;
      bfr[x] = *reinterpret_cast<const bf16x8*>(bs + rb2 * BK + tswz(rb2, j) * 8);
    }
#pragma unroll
    for (int x = 0; x < 8; ++x)
#pragma unroll
      for (int y = 0; y < 8; ++y)
        acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[x], bfr[y], acc[x][y], 0, 0, 0);
  }

  // Epilogue. acc[x][y][i] = C[row0 + 128 wm + 16x + 4j + i][col0 + 128 wn + 16y + m].
  const int head = (col0 + 128 * wn) / DH;  // 0..2*Hkv-1: K heads first, then V heads
  const bool is_k = head < a.hkv;
  bf16* dst_base = is_k ? a.k_out : a.v_out;
  const int hh = is_k ? head : head - a.hkv;
  float kw[8];
#pragma unroll
  for (int y = 0; y < 8; ++y) kw[y] = a.knw[16 * y + m];
#pragma unroll
  for (int x = 0; x < 8; ++x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = row0 + 128 * wm + 16 * x + 4 * j + i;
      const bool rv = row < a.rows;
      const float rs = rv ? a.rstd[row] : 0.f;
      float y8[8];
#pragma unroll
      for (int y = 0; y < 8; ++y) y8[y] = acc[x][y][i] * rs;
      if (is_k) {
        float ss = 0.f;
#pragma unroll
        for (int y = 0; y < 8; ++y) ss += y8[y] * y8[y];
        ss = group_sum<16>(ss);  // the 16 lanes of group j hold this row's 128 columns
        const float inv = 1.0f / sqrtf(ss * (1.0f / DH) + a.eps);
#pragma unroll
        for (int y = 0; y < 8; ++y) y8[y] *= inv * kw[y];
        if (rv) {
          int32_t p = a.pos[row];
          p = p < 0 ? 0 : (p >= a.max_pos ? a.max_pos - 1 : p);
          const float2* cs = a.table + (int64_t)p * HALF + m;
#pragma unroll
          for (int y = 0; y < 4; ++y) {
            const float2 c = cs[16 * y];
            const float lo = y8[y], hi = y8[y + 4];
            y8[y] = lo * c.x - hi * c.y;
            y8[y + 4] = hi * c.x + lo * c.y;
          }
        }
      }
      if (rv) {
        bf16* dst = dst_base + (row * a.hkv + hh) * DH + m;
#pragma unroll
        for (int y = 0; y < 8; ++y) dst[16 * y] = f2bf(y8[y]);
      }
    }
  }
}

}  // namespace

size_t context_kv_workspace_bytes(int64_t rows, int32_t hidden, int32_t hkv, int32_t dh) {
  return align256((size_t)2 * hkv * dh * hidden * sizeof(bf16)) + align256((size_t)rows * sizeof(float));
}

hipError_t launch_context_kv(const void* hidden, const float* hnw, const void* wk,
                             const void* wv, const float* knw, const int32_t* pos, int64_t rows,
                             int32_t hidden_size, int32_t hkv, int32_t dh, float eps,
                             const float* table, int32_t max_pos, void* k_out, void* v_out,
                             void* ws, hipStream_t s) {
  const int64_t kdim = (int64_t)hkv * dh;
  bf16* wfold = (bf16*)ws;
  float* rstd = (float*)((char*)ws + align256((size_t)2 * kdim * hidden_size * sizeof(bf16)));
  {
    const int64_t n8 = 2 * kdim * hidden_size / 8;
    hipLaunchKernelGGL(fold_weights_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s,
                       (const bf16*)wk, (const bf16*)wv, hnw, wfold, kdim, hidden_size);
  }
  hipLaunchKernelGGL(row_rstd_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s,
                     (const bf16*)hidden, rstd, rows, hidden_size, eps);
  CkvArgs a{};
  a.h = (const bf16*)hidden;
  a.w = wfold;
  a.rstd = rstd;
  a.knw = knw;
  a.pos = pos;
  a.table = reinterpret_cast<const float2*>(table);
  a.k_out = (bf16*)k_out;
  a.v_out = (bf16*)v_out;
  a.rows = rows;
  a.hidden = hidden_size;
  a.n = (int32_t)(2 * kdim);
  a.hkv = hkv;
  a.max_pos = max_pos;
  a.eps = eps;
  const int64_t mtiles = (rows + BM - 1) / BM;
  const int64_t blocks = (mtiles + 7) / 8 * 8 * (a.n / BN);  // whole groups of 8 row blocks
  const size_t lds = (size_t)NSTAGE * 2 * BM * BK * sizeof(bf16);
  static std::once_flag once[64];
  int dev = 0;
  (void)hipGetDevice(&dev);
  std::call_once(once[dev & 63], [] {
    (void)hipFuncSetAttribute((const void*)ctx_kv_gemm_kernel,
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              NSTAGE * 2 * BM * BK * (int)sizeof(bf16));
  });
  if (blocks > 0)
    hipLaunchKernelGGL(ctx_kv_gemm_kernel, dim3((unsigned)blocks), dim3(NT), lds, s, a);
  return hipGetLastError();
}

}  // namespace dflash
