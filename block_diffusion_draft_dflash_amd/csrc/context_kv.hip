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
// applied in the GEMM epilogue; the GEMM computes it from the A fragments
// its waves already hold (no separate pass over the hidden states). The GEMM (M = rows, N = 2 * Hkv * Dh, K = H)
// runs on v_mfma_f32_16x16x32_bf16 with 256x256 workgroup tiles of 8 waves
// (two per SIMD); a wave owns 128 rows x 64 columns of one 128-wide head,
// chosen so that the rotate-half pairs (d, d + 64) meet in one lane; the
// k-norm's sum of squares is completed with the partner wave through LDS.
// The k-slices of A and B are copied HBM -> LDS directly (no register
// staging) up to NSTAGE slices ahead, with explicit waits and fence-free
// barriers, and each wave reads the next slice's fragments while the MFMAs
// of the current one run.
#include <mutex>

#include "dflash_device.h"
#include "dflash_internal.h"

namespace dflash {
namespace {

constexpr int BM = 256, BN = 256, BK = 32;

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

struct CkvArgs {
  const bf16* h;        // [rows, H]
  const bf16* w;        // [N, H] folded weights, K rows then V rows
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
// chunk c of row r is stored at c ^ ((r >> 1) & 3). A fragment read (16
// consecutive rows at one logical chunk) is served 8 lanes = 128 bytes at a
// time; rows 2i and 2i + 1 share a 128-byte line at offsets 0 and 64, and the
// XOR moves each pair of the 8 rows to its own 16-byte slot, so the 8 lanes hit
// distinct banks. (The former c ^ ((r >> 2) & 3) put rows r and r + 2 in the
// same banks: 48% of the GEMM's LDS cycles were bank conflicts.)
__device__ __forceinline__ int tswz(int row, int c) { return c ^ ((row >> 1) & 3); }

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

constexpr int NTG = 512;  // GEMM workgroup: 8 waves, two per SIMD

__global__ __launch_bounds__(NTG) void ctx_kv_gemm_kernel(CkvArgs a) {
  constexpr int DH = 128;
  constexpr int HALF = DH / 2;
  constexpr int TILE = BM * BK;               // elements per A (or B) k-slice
  constexpr int NW = NTG / 64;
  constexpr int CPW = TILE / 512 / NW;        // 1 KB copies per wave per operand per k-slice (2)
  constexpr int CPS = 2 * CPW;                // per thread per k-slice (A and B)
  extern __shared__ __attribute__((aligned(16))) bf16 smem[];  // [stage][A | B]

  // Block order: the dispatcher deals workgroups to the 8 XCDs round-robin.
  // Consecutive row blocks go to different XCDs and each XCD runs all column
  // tiles of its row blocks.
  const int ntn = a.n / BN;
  const int xcd = blockIdx.x % 8;
  const int slot = blockIdx.x / 8;
  const int64_t rb = (int64_t)(slot / ntn) * 8 + xcd;
  const int64_t row0 = rb * BM;
  if (row0 >= a.rows) return;
  const int col0 = (slot % ntn) * BN;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, m = lane & 15, j = lane >> 4;
  // Wave tile: 128 rows (half wm) x 64 columns of head hw of the tile: the
  // 32-column chunks cc and cc + 2 of the head (columns d and d + 64 of a
  // rotate-half pair are in the same lane); the partner wave (w ^ 2) holds
  // the head's other 64 columns.
  const int wm = w & 1, wn = w >> 1, hw = wn >> 1, cc = wn & 1;
  auto hcol = [&](int y) { return (y >> 1) * HALF + cc * 32 + (y & 1) * 16; };  // column in head

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

  f32x4 acc[8][4];
#pragma unroll
  for (int x = 0; x < 8; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto read_frags = [&](int32_t ks, bf16x8 (&af)[8], bf16x8 (&bfr)[4]) {
    const bf16* as = smem + (ks % NSTAGE) * 2 * TILE;
    const bf16* bs = as + TILE;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const int ra = 128 * wm + 16 * x + m;
      af[x] = *reinterpret_cast<const bf16x8*>(as + ra * BK + tswz(ra, j) * 8);
    }
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int rbb = hw * DH + hcol(y) + m;
      bfr[y] = *reinterpret_cast<const bf16x8*>(bs + rbb * BK + tswz(rbb, j) * 8);
    }
  };
  auto mma = [&](const bf16x8 (&af)[8], const bf16x8 (&bfr)[4]) {
#pragma unroll
    for (int x = 0; x < 8; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y)
        acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[x], bfr[y], acc[x][y], 0, 0, 0);
  };
  // wait until this thread's copies of slice t landed, given the last slice issued
  auto wait_slice = [&](int32_t t, int32_t last) {
    const int32_t after = min(last - t, NSTAGE - 1);
    if (after >= 3) wait_vmcnt<3 * CPS>();
    else if (after == 2) wait_vmcnt<2 * CPS>();
    else if (after == 1) wait_vmcnt<CPS>();
    else wait_vmcnt<0>();
  };
  auto lgkm0 = [] { __builtin_amdgcn_s_waitcnt(0xC07F); };

  const int32_t ksteps = a.hidden / BK;
  auto read_a = [&](int32_t ks, bf16x8 (&af)[8]) {
    const bf16* as = smem + (ks % NSTAGE) * 2 * TILE;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const int ra = 128 * wm + 16 * x + m;
      af[x] = *reinterpret_cast<const bf16x8*>(as + ra * BK + tswz(ra, j) * 8);
    }
  };
  auto read_b = [&](int32_t ks, bf16x8 (&bfr)[4]) {
    const bf16* bs = smem + (ks % NSTAGE) * 2 * TILE + TILE;
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int rbb = hw * DH + hcol(y) + m;
      bfr[y] = *reinterpret_cast<const bf16x8*>(bs + rbb * BK + tswz(rbb, j) * 8);
    }
  };
  int32_t last = -1;
#pragma unroll
  for (int t = 0; t < NSTAGE; ++t)
    if (t < ksteps) { issue(t); last = t; }
  bf16x8 fa[8], fb[4], gb[4];
  float hsq[2] = {0.f, 0.f};  // hidden row sums of squares, row blocks 2wn and 2wn + 1
  wait_slice(0, last);
  block_barrier();
  read_b(0, fb);
  for (int32_t ks = 0; ks < ksteps; ++ks) {
    read_a(ks, fa);
    // B of slice ks in fb; A of slice ks read above; B of ks+1 under the MFMAs
    if (ks + 1 < ksteps) {
      wait_slice(ks + 1, last);
      lgkm0();
      block_barrier();
      if (ks + NSTAGE < ksteps) { issue(ks + NSTAGE); last = ks + NSTAGE; }
      read_b(ks + 1, gb);
    }
    mma(fa, fb);
    // the four waves that share these A rows split the row sums: wave wn takes
    // row blocks 2wn, 2wn + 1 (selected without dynamic register indexing)
#pragma unroll
    for (int x = 0; x < 8; ++x)
      if ((x >> 1) == wn) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = bf2f(fa[x][e]);
          hsq[x & 1] += v * v;
        }
      }
#pragma unroll
    for (int y = 0; y < 4; ++y) fb[y] = gb[y];
  }

  // Row scale of the hidden RMSNorm, from the A fragments the waves consumed:
  // 1 / sqrt(mean(h^2) + eps) per row, shared through LDS.
  float* rst = reinterpret_cast<float*>(smem) + NW * 128;  // [256]
  lgkm0();
  block_barrier();  // every wave is done with the stages
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float ss = xrow4_sum(hsq[h]);  // the 4 lane groups cover the row's k chunks
    if (j == 0) rst[128 * wm + 16 * (2 * wn + h) + m] = 1.0f / sqrtf(ss / (float)a.hidden + a.eps);
  }
  lgkm0();
  block_barrier();
  // Epilogue. acc[x][y][i] = C[row0 + 128 wm + 16x + 4j + i][col0 + 128 hw + hcol(y) + m].
  const int head = (col0 + DH * hw) / DH;  // 0..2*Hkv-1: K heads first, then V heads
  const bool is_k = col0 < a.hkv * DH;     // a 256-column tile is all K or all V
  bf16* dst_base = is_k ? a.k_out : a.v_out;
  const int hh = is_k ? head : head - a.hkv;
  if (is_k) {
    // per-head RMSNorm: this wave's 64 columns of each row, then the partner's
    float* sq = reinterpret_cast<float*>(smem);  // [NW][128]
#pragma unroll
    for (int x = 0; x < 8; ++x)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t row = row0 + 128 * wm + 16 * x + 4 * j + i;
        const float rs = row < a.rows ? rst[128 * wm + 16 * x + 4 * j + i] : 0.f;
        float ss = 0.f;
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          const float v = acc[x][y][i] * rs;
          ss += v * v;
        }
        ss = group_sum<16>(ss);  // the 16 lanes of group j hold this row's 64 columns
        if (m == 0) sq[w * 128 + 16 * x + 4 * j + i] = ss;
      }
    lgkm0();
    block_barrier();
  }
  float kw[4];
#pragma unroll
  for (int y = 0; y < 4; ++y) kw[y] = a.knw[hcol(y) + m];
#pragma unroll
  for (int x = 0; x < 8; ++x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rloc = 16 * x + 4 * j + i;
      const int64_t row = row0 + 128 * wm + rloc;
      const bool rv = row < a.rows;
      const float rs = rv ? rst[rloc + 128 * wm] : 0.f;
      float y4[4];
#pragma unroll
      for (int y = 0; y < 4; ++y) y4[y] = acc[x][y][i] * rs;
      if (is_k) {
        const float* sq = reinterpret_cast<const float*>(smem);
        const float ss = sq[w * 128 + rloc] + sq[(w ^ 2) * 128 + rloc];
        const float inv = 1.0f / sqrtf(ss * (1.0f / DH) + a.eps);
#pragma unroll
        for (int y = 0; y < 4; ++y) y4[y] *= inv * kw[y];
        if (rv) {
          int32_t p = a.pos[row];
          p = p < 0 ? 0 : (p >= a.max_pos ? a.max_pos - 1 : p);
          const float2* cs = a.table + (int64_t)p * HALF;
#pragma unroll
          for (int y = 0; y < 2; ++y) {  // pairs (d, d + 64): y and y + 2
            const float2 c = cs[hcol(y) + m];
            const float lo = y4[y], hi = y4[y + 2];
            y4[y] = lo * c.x - hi * c.y;
            y4[y + 2] = hi * c.x + lo * c.y;
          }
        }
      }
      if (rv) {
        bf16* dst = dst_base + (row * a.hkv + hh) * DH + m;
#pragma unroll
        for (int y = 0; y < 4; ++y) dst[hcol(y)] = f2bf(y4[y]);
      }
    }
  }
}

}  // namespace

size_t context_kv_workspace_bytes(int64_t rows, int32_t hidden, int32_t hkv, int32_t dh) {
  (void)rows;
  return align256((size_t)2 * hkv * dh * hidden * sizeof(bf16));
}

hipError_t launch_context_kv(const void* hidden, const float* hnw, const void* wk,
                             const void* wv, const float* knw, const int32_t* pos, int64_t rows,
                             int32_t hidden_size, int32_t hkv, int32_t dh, float eps,
                             const float* table, int32_t max_pos, void* k_out, void* v_out,
                             void* ws, hipStream_t s) {
  const int64_t kdim = (int64_t)hkv * dh;
  bf16* wfold = (bf16*)ws;
  {
    const int64_t n8 = 2 * kdim * hidden_size / 8;
    hipLaunchKernelGGL(fold_weights_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s,
                       (const bf16*)wk, (const bf16*)wv, hnw, wfold, kdim, hidden_size);
  }

  CkvArgs a{};
  a.h = (const bf16*)hidden;
  a.w = wfold;
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
    hipLaunchKernelGGL(ctx_kv_gemm_kernel, dim3((unsigned)blocks), dim3(NTG), lds, s, a);
  return hipGetLastError();
}

}  // namespace dflash
