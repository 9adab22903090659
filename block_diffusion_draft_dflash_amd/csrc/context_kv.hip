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
// its waves already hold (no separate pass over the hidden states). The GEMM
// (M = rows, N = 2 * Hkv * Dh, K = H) runs on v_mfma_f32_32x32x16_bf16 with
// its accumulators in AGPRs, in 256x256 workgroup tiles of 4 waves (one per
// SIMD); a wave owns 128 rows x one whole 128-wide head, so the k-norm and
// the rotate-half pairs (d, d + 64) stay inside the wave. The 64-wide
// k-slices of A and B are copied HBM -> LDS directly (no register staging),
// the next slice in flight while the current one is consumed, with explicit
// waits and one fence-free barrier per slice; each wave's fragment reads are
// interleaved with its MFMAs. The products are formed transposed (weights as
// the first operand), so each lane ends up with four consecutive columns of
// its rows: the epilogue completes a row's k-norm with one cross-lane add,
// reads the rows' cos/sin from LDS (copied there once per tile) and stores
// 8-byte pieces of the output rows straight from registers.
#include <mutex>

#include "dflash_device.h"
#include "dflash_internal.h"

namespace dflash {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;

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

// A and B k-stages are [256 rows][64 k] bf16 (128-byte rows, 8 chunks of
// 16 B); chunk c of row r is stored at c ^ ((r >> 1) & 7). A 32x32x16
// fragment read takes 32 consecutive rows at logical chunk c (lanes 0-31) and
// c + 1 (lanes 32-63); with this swizzle the read has no bank conflicts
// (measured with the LDS bank-conflict counter).
__device__ __forceinline__ int tswz(int row, int c) { return c ^ ((row >> 1) & 7); }

#ifndef SCHED_CORE
#define SCHED_CORE 1
#endif
constexpr int NSTAGE = 2;  // LDS stages of 64-k (A, B) slices: the next one in flight

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14; expcnt and lgkmcnt left at their no-wait maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// Workgroup barrier without the memory fence of __syncthreads() (which would
// drain the k-slices still in flight).
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

constexpr int NTG = 256;  // GEMM workgroup: 4 waves, one per SIMD

// One workgroup computes a 256-row x 256-column tile (two heads) of
// [K | V] = h W'^T over the whole of H. Wave w owns rows 128 (w & 1) ..+127
// and head (w >> 1) of the tile: 4 x 4 blocks of 32 x 32 outputs (formed as
// W' h^T, so that a lane holds row elements) on
// v_mfma_f32_32x32x16_bf16, whose 256 f32 accumulators per lane sit in the
// accumulation registers. (Back to back on register operands the 32x32x16
// and 16x16x32 forms run within 5% of each other on this GPU, ~1.8-1.9
// PFLOP/s on random data and ~2.2-2.3 on zeros; the 32x32 form needs 16
// independent accumulators per wave where the 16x16 one needs 64.)
// Each 64-k stage is consumed as two 32-k sub-slices: per sub-slice a wave
// reads 8 A and 8 B fragments from LDS (16 KB) for 32 MFMAs, the next
// sub-slice's fragments being read, and the current A fragments' squares
// summed for the row norm, in between those MFMAs. One barrier per stage.
// The body is instantiated per head of the tile (WN, the waves' w >> 1) so
// that each wave's share of the row-norm sums (k-half WN of every sub-slice)
// selects its fragments at compile time.
template <int WN>
__device__ __forceinline__ void ctx_kv_gemm_body(const CkvArgs& a, bf16* smem) {
  constexpr int DH = 128;
  constexpr int HALF = DH / 2;
  constexpr int TILE = BM * BK;               // elements per A (or B) stage
  constexpr int NW = NTG / 64;
  constexpr int CPW = TILE / 512 / NW;        // 1 KB copies per wave per operand per stage (8)

  // Block order: the dispatcher deals workgroups to the 8 XCDs round-robin.
  // Consecutive row blocks go to different XCDs and each XCD runs all column
  // tiles of its row blocks together (they read the same A slices).
  const int ntn = a.n / BN;
  const int xcd = blockIdx.x % 8;
  const int slot = blockIdx.x / 8;
  const int64_t rb = (int64_t)(slot / ntn) * 8 + xcd;
  const int64_t row0 = rb * BM;
  if (row0 >= a.rows) return;
  const int col0 = (slot % ntn) * BN;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;  // MFMA row / column within a block, lane half
  const int wm = w & 1;
  constexpr int wn = WN;

  // Copy sources: a scalar base per operand (the workgroup's first row, then
  // advanced one stage per copy) and a 32-bit byte offset per lane and copy:
  // a 1 KB copy fills 8 rows of 128 bytes, lane l row l / 8 at logical chunk
  // tswz(row, l % 8).
  const bf16* abase = a.h + row0 * a.hidden;
  const bf16* bbase = a.w + (int64_t)col0 * a.hidden;
  // (B has no partial tiles: its offset is a lane part, which depends on the
  // copy's parity only, plus a uniform part folded into the base)
  uint32_t aoff[CPW], boff[2];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int r = (w * CPW + i) * 8 + lane / 8;
    const int c = tswz(r, lane % 8);
    const int ra = (int)min((int64_t)r, a.rows - 1 - row0);  // rows past the end re-read the last
    aoff[i] = (uint32_t)(ra * a.hidden + c * 8) * 2u;
    if (i < 2) boff[i] = (uint32_t)(r * a.hidden + c * 8) * 2u;
  }
  // LDS byte address of the dynamic shared memory (uniform)
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(DF_LDS void*)smem);
  auto dma = [](const bf16* base, uint32_t voff, uint32_t lds_addr) {
    // the base is uniform; say so, so that it sits in scalar registers
    const uint64_t b = (uint64_t)(uintptr_t)base;
    const uint64_t sb = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds_addr), "v"(voff), "s"(sb)
                 : "memory", "m0");
  };
  constexpr uint32_t STAGE_BYTES = 2 * TILE * sizeof(bf16);
  auto issue = [&](int32_t st_idx) {
    const uint32_t st = lds0 + (uint32_t)(st_idx % NSTAGE) * STAGE_BYTES;
    const int32_t k0 = st_idx * BK;
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      dma(abase + k0, aoff[i], st + (w * CPW + i) * 1024);
      dma(bbase + k0 + (int64_t)(i & ~1) * 8 * a.hidden, boff[i & 1], st + TILE * 2 + (w * CPW + i) * 1024);
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[x][y][e] = 0.f;

  // Fragment (x, h) of sub-slice j of A: rows 128 wm + 32 x + l32, k 32 j +
  // 16 h + 8 hi .. +7 of the stage (logical chunk 4 j + 2 h + hi); B likewise
  // over rows 128 wn + 32 y + l32. The swizzle depends on l32 only, so each
  // (operand, j, h) has one per-lane base and the blocks sit at fixed offsets.
  int a_lane[2][2], b_lane[2][2];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      a_lane[jj][h] = (128 * wm + l32) * BK + tswz(l32, 4 * jj + 2 * h + hi) * 8;
      b_lane[jj][h] = TILE + (128 * wn + l32) * BK + tswz(l32, 4 * jj + 2 * h + hi) * 8;
    }
  auto frag = [&](int32_t st_idx, int lane_off, int x) {
    const bf16* p = smem + (st_idx % NSTAGE) * 2 * TILE + lane_off;
    return *reinterpret_cast<const bf16x8*>(p + x * 32 * BK);
  };
  const int32_t nst = a.hidden / BK;  // stages (H is a multiple of 64)

  // hidden row sums of squares of rows 128 wm + 32 x + l32, this wave's share:
  // k-half WN of every sub-slice (the other head's wave takes the other half),
  // one bf16 dot product per pair of elements, into two independent partial
  // sums per row so that no dot product waits for the previous one
  float hsq[4][2] = {{0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}};
  auto row_sum_part = [&](const bf16x8& v8, int x, int half) {
#pragma unroll
    for (int e = 2 * half; e < 2 * half + 2; ++e) {
      const bf16x2 p2 = {v8[2 * e], v8[2 * e + 1]};
      hsq[x][e & 1] = __builtin_amdgcn_fdot2_f32_bf16(p2, p2, hsq[x][e & 1], false);
    }
  };
  // fragments of one sub-slice: [0..3] B blocks at k-half 0, [4..7] at k-half
  // 1 (read first, every MFMA needs them), then A likewise
  auto read_frag = [&](int32_t st_idx, int jj, int q, bf16x8 (&na)[8], bf16x8 (&nb)[8]) {
    if (q < 8) nb[q] = frag(st_idx, b_lane[jj][q >> 2], q & 3);
    else na[q - 8] = frag(st_idx, a_lane[jj][(q - 8) >> 2], (q - 8) & 3);
  };
  // The weight block goes in as the first operand and the hidden block as the
  // second, so that the accumulators come out transposed: lane (l32, hi)
  // holds row 32 x + l32 of block (x, y) at the four consecutive columns
  // 32 y + 8 q + 4 hi .. +3 for q = e / 4 (see the epilogue).
  auto mma = [&](const bf16x8 (&ca)[8], const bf16x8 (&cb)[8], int x, int h, int y) {
    acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cb[4 * h + y], ca[4 * h + x], acc[x][y],
                                                        0, 0, 0);
  };
  // The 32 MFMAs of one sub-slice on (ca, cb), with the 16 fragment reads of
  // the next sub-slice (stage st_idx, half jj) into (na, nb) between them.
  auto core = [&](const bf16x8 (&ca)[8], const bf16x8 (&cb)[8], bf16x8 (&na)[8],
                  bf16x8 (&nb)[8], int32_t st_idx, int jj) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int x = q >> 2, h = (q >> 1) & 1, y0 = 2 * (q & 1);
      read_frag(st_idx, jj, q, na, nb);
      mma(ca, cb, x, h, y0);
      mma(ca, cb, x, h, y0 + 1);
    }
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      row_sum_part(ca[4 * WN + x], x, 0);
      row_sum_part(ca[4 * WN + x], x, 1);
    }
#if SCHED_CORE
    // one fragment read per two MFMAs: at most a few LDS reads outstanding at
    // any time (the LDS counter holds 15), none of them holding up an MFMA
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);  // 1 VALU
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
    }
#endif
  };
  auto core_last = [&](const bf16x8 (&ca)[8], const bf16x8 (&cb)[8]) {
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int y = 0; y < 4; ++y) mma(ca, cb, x, h, y);
        if (h == WN) {
          row_sum_part(ca[4 * h + x], x, 0);
          row_sum_part(ca[4 * h + x], x, 1);
        }
      }
  };

  // K tiles: the positions of the tile's rows (thread t: row t), loaded ahead
  // of the slices so that the epilogue does not wait for them.
  const bool is_k = col0 < a.hkv * DH;  // a 256-column tile is all K or all V
  int32_t my_pos = 0;
  if (is_k) my_pos = a.pos[min(row0 + tid, a.rows - 1)];

  bf16x8 fa[8], fb[8], ga[8], gb[8];
  issue(0);
  if (nst > 1) {
    issue(1);
    wait_vmcnt<2 * CPW>();  // stage 0 landed (stage 1 may stay in flight)
  } else {
    wait_vmcnt<0>();
  }
  block_barrier();
#pragma unroll
  for (int q = 0; q < 16; ++q) read_frag(0, 0, q, fa, fb);
  for (int32_t st = 0; st + 1 < nst; ++st) {
    // first half of stage st, while its second half's fragments are read
    core(fa, fb, ga, gb, st, 1);
    // stage st + 1 landed everywhere, and every wave's reads of stage st are
    // done: stage st's buffer takes stage st + 2
    wait_vmcnt<0>();
    wait_lgkm0();
    block_barrier();
    if (st + 2 < nst) issue(st + 2);
    core(ga, gb, fa, fb, st + 1, 0);
  }
  core(fa, fb, ga, gb, nst - 1, 1);  // the last stage
  core_last(ga, gb);

  // Epilogue. After the slices the LDS holds, from its start: the cos/sin
  // rows of the tile's 256 rows (K tiles; row t at t * CS_STRIDE bytes), then
  // the two waves' partial row sums, the row scales and the clamped positions.
  // The cos/sin rows are 16 bytes further apart than their 512 bytes, so that
  // the 32 lanes reading one offset of 32 consecutive rows hit distinct banks.
  constexpr int CS_STRIDE = HALF * 8 + 16;
  char* const lds_b = reinterpret_cast<char*>(smem);
  float* rpart = reinterpret_cast<float*>(lds_b + 256 * CS_STRIDE);  // [2][256]
  float* rsc = rpart + 512;                                          // [256] row scales
  int32_t* rpos = reinterpret_cast<int32_t*>(rsc + 256);             // [256] clamped positions
  const int head = (col0 + DH * wn) / DH;  // 0..2*Hkv-1: K heads first, then V heads
  const int hh = is_k ? head : head - a.hkv;
  bf16* dst_base = is_k ? a.k_out : a.v_out;
  // the k-norm weights of this lane's columns 32 y + 8 q + 4 hi .. +3
  float4 kwv[4][4];
  if (is_k) {
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
      for (int q = 0; q < 4; ++q) kwv[y][q] = *reinterpret_cast<const float4*>(a.knw + 32 * y + 8 * q + 4 * hi);
  }
  wait_lgkm0();
  block_barrier();  // every wave is done with the stages
  // Row scale of the hidden RMSNorm, 1 / sqrt(mean(h^2) + eps): the two
  // waves' partial sums of each row meet in LDS, with the rows' positions.
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const float ss = hsq[x][0] + hsq[x][1];
    const float s2 = ss + __shfl_xor(ss, 32, 64);  // both lane halves' k chunks
    if (hi == 0) rpart[256 * WN + 128 * wm + 32 * x + l32] = s2;
  }
  rpos[tid] = my_pos < 0 ? 0 : (my_pos >= a.max_pos ? a.max_pos - 1 : my_pos);
  wait_lgkm0();
  block_barrier();
  if (is_k) {
    // the cos/sin row of each of the tile's rows, HBM -> LDS: one 512-byte
    // copy per row (32 lanes of 16 bytes), wave w taking rows 64 w .. 64 w + 63
    for (int i = 0; i < 64; ++i) {
      const int r = 64 * w + i;
      const uint32_t dst = lds0 + (uint32_t)(r * CS_STRIDE);
      if (lane < 32) {
        const float2* src = a.table + (int64_t)rpos[r] * HALF + 2 * lane;
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                     :
                     : "s"(dst), "v"(src)
                     : "memory", "m0");
      }
    }
  }
  rsc[tid] = 1.0f / sqrtf((rpart[tid] + rpart[256 + tid]) / (float)a.hidden + a.eps);
  wait_vmcnt<0>();  // this wave's cos/sin copies (and the weights) landed
  wait_lgkm0();
  block_barrier();  // every wave's copies and row scales are visible

  // acc[x][y][e] = C[row0 + 128 wm + 32 x + l32][col0 + 128 wn + 32 y + 8 (e / 4) + 4 hi + e % 4]:
  // each lane holds 64 of a row's 128 columns of this head (the other 64 in
  // lane l ^ 32), the rotate-half pairs (d, d + 64) = blocks (y, y + 2) in
  // the same lane, and writes whole 8-byte pieces of the output row.
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int rt = 128 * wm + 32 * x + l32;  // row within the tile
    const int64_t row = row0 + rt;
    const float rs = rsc[rt];
    float v[4][16];
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
      for (int e = 0; e < 16; ++e) v[y][e] = acc[x][y][e] * rs;
    if (is_k) {
      float ss = 0.f;
#pragma unroll
      for (int y = 0; y < 4; ++y)
#pragma unroll
        for (int e = 0; e < 16; ++e) ss += v[y][e] * v[y][e];
      ss += __shfl_xor(ss, 32, 64);  // the row's other 64 columns
      const float inv = 1.0f / sqrtf(ss * (1.0f / DH) + a.eps);
      const char* csrow = lds_b + rt * CS_STRIDE;
#pragma unroll
      for (int y = 0; y < 2; ++y)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // cos/sin of dims d = 32 y + 8 q + 4 hi .. +3 (pairs (d, d + 64))
          const f32x4 c01 = *reinterpret_cast<const f32x4*>(csrow + (32 * y + 8 * q + 4 * hi) * 8);
          const f32x4 c23 = *reinterpret_cast<const f32x4*>(csrow + (32 * y + 8 * q + 4 * hi) * 8 + 16);
          const float cs[8] = {c01[0], c01[1], c01[2], c01[3], c23[0], c23[1], c23[2], c23[3]};
          const float4 w0 = kwv[y][q], w1 = kwv[y + 2][q];
          const float wlo[4] = {w0.x, w0.y, w0.z, w0.w}, whi[4] = {w1.x, w1.y, w1.z, w1.w};
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int e = 4 * q + r4;
            const float lo = v[y][e] * inv * wlo[r4], hi2 = v[y + 2][e] * inv * whi[r4];
            const float c = cs[2 * r4], sn = cs[2 * r4 + 1];
            v[y][e] = lo * c - hi2 * sn;
            v[y + 2][e] = hi2 * c + lo * sn;
          }
        }
    }
    if (row < a.rows) {
      bf16* drow = dst_base + (row * a.hkv + hh) * DH + 4 * hi;
#pragma unroll
      for (int y = 0; y < 4; ++y)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          bf16x4 o;
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) o[r4] = f2bf(v[y][4 * q + r4]);
          *reinterpret_cast<bf16x4*>(drow + 32 * y + 8 * q) = o;
        }
    }
  }
}

__global__ __launch_bounds__(NTG) __attribute__((amdgpu_waves_per_eu(1, 1)))
void ctx_kv_gemm_kernel(CkvArgs a) {
  extern __shared__ __attribute__((aligned(16))) bf16 smem[];  // [stage][A | B]
  if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 7) == 0) ctx_kv_gemm_body<0>(a, smem);
  else ctx_kv_gemm_body<1>(a, smem);
}

// LDS of the GEMM: the k-slice stages, or in the epilogue the cos/sin rows
// of the tile's rows, the partial row sums, row scales and positions,
// whichever is larger.
constexpr size_t kEpiLds = (size_t)256 * (64 * 8 + 16) + 4096;
constexpr size_t kGemmLds = (size_t)NSTAGE * 2 * BM * BK * sizeof(bf16) > kEpiLds
                                ? (size_t)NSTAGE * 2 * BM * BK * sizeof(bf16)
                                : kEpiLds;

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
  const int64_t fold_blocks = (2 * kdim * hidden_size / 8 + 255) / 256;
  const int64_t mtiles = (rows + BM - 1) / BM;
  const int64_t blocks = (mtiles + 7) / 8 * 8 * (2 * kdim / BN);  // whole groups of 8 row blocks
  if (!grid_fits(fold_blocks) || !grid_fits(blocks)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(fold_weights_kernel, dim3((unsigned)fold_blocks), dim3(256), 0, s,
                     (const bf16*)wk, (const bf16*)wv, hnw, wfold, kdim, hidden_size);

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
  const size_t lds = kGemmLds;
  static std::once_flag once[64];
  int dev = 0;
  (void)hipGetDevice(&dev);
  std::call_once(once[dev & 63], [] {
    (void)hipFuncSetAttribute((const void*)ctx_kv_gemm_kernel,
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)kGemmLds);
  });
  if (blocks > 0)
    hipLaunchKernelGGL(ctx_kv_gemm_kernel, dim3((unsigned)blocks), dim3(NTG), lds, s, a);
  return hipGetLastError();
}

}  // namespace dflash
