// The draft layer's projections around the block attention.
//
// "qwen3_dflash.cpp" page, ForwardBlockLogits and ForwardWithCtxKVDev:
// input_layernorm is the standard residual add + RMSNorm (the residual stream
// becomes hidden + residual, the normed rows are a bf16 tensor), the normed
// block rows go through one product with the merged qkv weight whose row
// blocks are the q, k and v heads, and after the attention the output rows
// [T, Hq * Dh] go through the o_proj weight. Both products are x * W^T with
// W row-major [out, in].
//
// Kernels:
//   residual_norm_kernel  one workgroup per row: res = hidden (+ residual,
//                         stored back as bf16), normed = bf16(res * rstd * w).
//   proj_gemm_kernel      C[T, N] = A[T, K] * W[N, K]^T on bf16 MFMA with f32
//                         accumulation. A workgroup owns a 128 x 64 or 128 x 128
//                         output tile and a slice of K; K advances 64 at a time
//                         through a ring of LDS stages filled by direct HBM ->
//                         LDS copies (XOR-swizzled 128-byte rows, explicit
//                         waits). With few tiles (T ~ 128: the weights are the
//                         bytes) K is split so that every CU streams a share of
//                         the weight; the slices then write f32 partial tiles.
//   split_sum_kernel      sums the K-slice partials and rounds to bf16.
//   split_sum_krope_kernel  the same sum for a few context rows' stacked
//                         [K | V] product, plus the K heads' k-norm and RoPE.
// Output columns go to up to three row-major destinations (q | k | v).
#include <algorithm>
#include <mutex>

#include "dflash_device.h"
#include "dflash_internal.h"

namespace dflash {
namespace {

constexpr int GBM = 128;  // output rows per workgroup tile
constexpr int GBK = 64;   // K per ring stage (two MFMA k-steps of 32)
constexpr int GNT = 256;  // threads (4 waves; wave w owns rows 32 w .. 32 w + 31)
constexpr int A_TILE = GBM * GBK;
// Two tile shapes: 128 x 64 with 4 stages and 128 x 128 with 3 stages (both
// 96 KB of LDS, one workgroup per CU) for wide outputs. With the
// non-temporal weight copies these depths measured fastest: the wide tile
// with 3 stages against 2, 4 or 5, the narrow one with 4 against 3 or 5.
// Each stage copies the activation slice (A) next to the weight slice (W);
// the A slice is the same for every column tile, so a wider tile spends less
// of the bytes a CU keeps in flight on it.
template <int BN>
struct GemmShape {
  static constexpr int NS = BN == 128 ? 3 : 4;               // ring stages (NS - 1 in flight)
  static constexpr int W_TILE = BN * GBK;
  static constexpr int STAGE = A_TILE + W_TILE;              // bf16 elements per stage
  static constexpr int WCP = BN / 32;                        // W copies per wave per stage
  static constexpr int LPS = 4 + WCP;                        // copies per wave per stage
  static constexpr int CT = BN / 16;                         // 16-column tiles per wave
  static constexpr size_t LDS = (size_t)NS * STAGE * 2;
};
constexpr int NORM_MAX_CHUNKS = 4;  // 8-element chunks per thread in the row norm (H <= 8192)

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// s_waitcnt takes an immediate: at most k * STEP vector-memory operations
// outstanding, for a run-time k clamped to [0, MAXK].
template <int STEP, int MAXK>
__device__ __forceinline__ void wait_vmcnt_steps(int32_t k) {
  if constexpr (MAXK > 0) {
    if (k >= MAXK) {
      wait_vmcnt<MAXK * STEP>();
      return;
    }
    wait_vmcnt_steps<STEP, MAXK - 1>(k);
  } else {
    wait_vmcnt<0>();
  }
}
// Workgroup barrier without the fence of __syncthreads (which would drain the
// copies still in flight).
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// One wave-wide 16-byte-per-lane copy HBM -> LDS: lane l's 16 bytes land at
// dst + 16 l (dst is the wave's 1 KB destination). Issued from inline
// assembly so that the compiler does not drain it before every LDS read;
// every wait on it is explicit.
__device__ __forceinline__ void lds_copy16(const void* src, void* dst) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(DF_LDS void*)dst);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds), "v"(src)
               : "memory", "m0");
}
// The same copy with the non-temporal hint, for data read once per call (the
// weight slices): it streams through the caches instead of displacing the
// activations that every column tile re-reads.
__device__ __forceinline__ void lds_copy16_nt(const void* src, void* dst) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(DF_LDS void*)dst);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt"
               :
               : "s"(lds), "v"(src)
               : "memory", "m0");
}
// Physical 16-byte chunk of logical chunk c in a 128-byte LDS row.
__device__ __forceinline__ int swz(int row, int c) { return c ^ (row & 7); }

struct OutSegs {
  bf16* ptr[3];
  int64_t stride[3];  // elements between consecutive rows
  int32_t begin[4];   // segment s holds columns [begin[s], begin[s + 1])
};

__device__ __forceinline__ int seg_of(const OutSegs& o, int32_t n) {
  return n >= o.begin[2] ? 2 : (n >= o.begin[1] ? 1 : 0);
}

// ---------------------------------------------------------------------------
// input_layernorm: residual add + RMSNorm, one workgroup per row.
template <bool RES>
__global__ __launch_bounds__(256) void residual_norm_kernel(const bf16* __restrict__ hidden,
                                                            bf16* __restrict__ residual,
                                                            const float* __restrict__ w,
                                                            bf16* __restrict__ normed, int32_t H,
                                                            float eps) {
  // every argument in one batch of scalar loads (no dependent argument reads)
  asm volatile("" ::"s"(hidden), "s"(residual), "s"(w), "s"(normed), "s"(H), "s"(eps));
  __shared__ float red[4];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const int nch = H / 8;
  float x[NORM_MAX_CHUNKS][8];
  float4 wr[NORM_MAX_CHUNKS][2];  // the weights, loaded with the rows (one round trip)
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NORM_MAX_CHUNKS; ++i) {
    const int c = tid + 256 * i;
    if (c < nch) {
      wr[i][0] = *reinterpret_cast<const float4*>(w + 8 * c);
      wr[i][1] = *reinterpret_cast<const float4*>(w + 8 * c + 4);
    }
  }
#pragma unroll
  for (int i = 0; i < NORM_MAX_CHUNKS; ++i) {
    const int c = tid + 256 * i;
    if (c < nch) {
      const bf16x8 h = *reinterpret_cast<const bf16x8*>(hidden + t * H + 8 * c);
      if constexpr (RES) {
        // the residual stream becomes hidden + residual (stored as bf16);
        // the norm reads the stored value
        bf16x8* rp = reinterpret_cast<bf16x8*>(residual + t * H + 8 * c);
        const bf16x8 r = *rp;
        bf16x8 s;
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] = f2bf(bf2f(h[e]) + bf2f(r[e]));
        *rp = s;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[i][e] = bf2f(s[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[i][e] = bf2f(h[e]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += x[i][e] * x[i][e];
    }
  }
  ss = group_sum<64>(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  const float rstd = 1.0f / sqrtf(tot / (float)H + eps);
#pragma unroll
  for (int i = 0; i < NORM_MAX_CHUNKS; ++i) {
    const int c = tid + 256 * i;
    if (c < nch) {
      const float4 w0 = wr[i][0], w1 = wr[i][1];
      const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = f2bf(x[i][e] * rstd * wv[e]);
      *reinterpret_cast<bf16x8*>(normed + t * H + 8 * c) = o;
    }
  }
}

// ---------------------------------------------------------------------------
// C = A * W^T over one K slice of one 128 x BN tile.
struct GemmArgs {
  const bf16* a;   // [T, K]
  const bf16* w;   // rows [0, n1) of W: [n1, K]
  const bf16* w2;  // rows [n1, N) of W: [N - n1, K] (n1 a multiple of the tile width)
  int32_t n1;
  int64_t T;
  int32_t N, K;
  int32_t ksteps;  // GBK-steps per K slice (the last slice may be shorter)
  int32_t nsplit;
  float* part;  // [nsplit][T][N] f32 when nsplit > 1
  OutSegs out;
};

template <int BN>
__global__ __launch_bounds__(GNT) void proj_gemm_kernel(GemmArgs g) {
  using S = GemmShape<BN>;
  // the loader's arguments in one batch of scalar loads
  asm volatile("" ::"s"(g.a), "s"(g.w), "s"(g.w2), "s"(g.n1), "s"(g.T), "s"(g.N), "s"(g.K),
               "s"(g.ksteps), "s"(g.nsplit));
  extern __shared__ __attribute__((aligned(16))) bf16 smem[];
  const int32_t ntn = g.N / BN;
  int64_t id = blockIdx.x;
  const int32_t nt = (int32_t)(id % ntn);
  id /= ntn;
  const int32_t ks = (int32_t)(id % g.nsplit);
  const int64_t mt = id / g.nsplit;
  const int64_t m0 = mt * GBM;
  const int32_t n0 = nt * BN;
  const int32_t kbeg = ks * g.ksteps * GBK;
  const int32_t nk = max(0, min(g.ksteps, g.K / GBK - ks * g.ksteps));

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int m = lane & 15;
  const int j = lane >> 4;

  // Copy lanes: one wave-wide copy fills 8 rows of 128 bytes; lane l fetches
  // the logical chunk that the swizzle puts at (row l / 8, chunk l % 8).
  // Rows past T re-read row T - 1 (their results are never stored).
  const int r8 = lane >> 3, pc = lane & 7;
  int64_t a_src[4];
  int64_t w_src[S::WCP];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (w * 4 + i) * 8 + r8;
    const int64_t grow = min(m0 + row, g.T - 1);
    a_src[i] = grow * g.K + swz(row, pc) * 8;
  }
  // the tile's weight rows come from one of the two sources
  const bool second = n0 >= g.n1;
  const bf16* const wsrc = second ? g.w2 : g.w;
  const int32_t wn0 = second ? n0 - g.n1 : n0;
#pragma unroll
  for (int i = 0; i < S::WCP; ++i) {
    const int row = (w * S::WCP + i) * 8 + r8;
    w_src[i] = (int64_t)(wn0 + row) * g.K + swz(row, pc) * 8;
  }
  auto issue = [&](int32_t kt) {
    const int32_t k0 = kbeg + kt * GBK;
    bf16* st = smem + (kt % S::NS) * S::STAGE;
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_copy16(g.a + a_src[i] + k0, st + (w * 4 + i) * 8 * GBK);
#pragma unroll
    for (int i = 0; i < S::WCP; ++i)
      lds_copy16_nt(wsrc + w_src[i] + k0, st + A_TILE + (w * S::WCP + i) * 8 * GBK);
  };

  f32x4 acc[2][S::CT];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < S::CT; ++ct) acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int kt = 0; kt < S::NS - 1; ++kt)
    if (kt < nk) issue(kt);
  for (int32_t kt = 0; kt < nk; ++kt) {
    // own copies of stage kt landed (later stages may stay in flight); the
    // barrier makes every wave's part visible and frees stage kt - 1
    wait_vmcnt_steps<S::LPS, S::NS - 2>(nk - 1 - kt);
    block_barrier();
    if (kt + S::NS - 1 < nk) issue(kt + S::NS - 1);
    const bf16* st = smem + (kt % S::NS) * S::STAGE;
#pragma unroll
    for (int ss = 0; ss < 2; ++ss) {
      const int c = 4 * ss + j;  // logical 16-byte chunk (k = 8 c .. 8 c + 7)
      bf16x8 af[2], bf[S::CT];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const int row = 32 * w + 16 * rt + m;
        af[rt] = *reinterpret_cast<const bf16x8*>(st + row * GBK + swz(row, c) * 8);
      }
#pragma unroll
      for (int ct = 0; ct < S::CT; ++ct) {
        const int row = 16 * ct + m;
        bf[ct] = *reinterpret_cast<const bf16x8*>(st + A_TILE + row * GBK + swz(row, c) * 8);
      }
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < S::CT; ++ct)
          acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[rt], bf[ct], acc[rt][ct], 0, 0, 0);
    }
  }

  // lane (m, j): acc[rt][ct][i] = C[m0 + 32 w + 16 rt + 4 j + i][n0 + 16 ct + m]
  if (g.nsplit == 1) {
    const int sg = seg_of(g.out, n0);
    bf16* base = g.out.ptr[sg];
    const int64_t stride = g.out.stride[sg];
    const int32_t col = n0 - g.out.begin[sg];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t t = m0 + 32 * w + 16 * rt + 4 * j + i;
        if (t < g.T) {
#pragma unroll
          for (int ct = 0; ct < S::CT; ++ct) base[t * stride + col + 16 * ct + m] = f2bf(acc[rt][ct][i]);
        }
      }
  } else {
    float* p = g.part + (int64_t)ks * g.T * g.N;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t t = m0 + 32 * w + 16 * rt + 4 * j + i;
        if (t < g.T) {
#pragma unroll
          for (int ct = 0; ct < S::CT; ++ct) p[t * g.N + n0 + 16 * ct + m] = acc[rt][ct][i];
        }
      }
  }
}

// Sum of the K-slice partials, 8 columns a thread, in slice order. The
// partials of up to SB slices are loaded before any is added, so that their
// loads are in flight together (one memory round trip per SB slices).
constexpr int SB = 8;
__global__ __launch_bounds__(256) void split_sum_kernel(const float* __restrict__ part,
                                                        int32_t nsplit, int64_t T, int32_t N,
                                                        OutSegs out) {
  // every argument in one batch of scalar loads (no dependent argument reads)
  asm volatile("" ::"s"(part), "s"(nsplit), "s"(T), "s"(N), "s"(out.ptr[0]), "s"(out.ptr[1]),
               "s"(out.ptr[2]), "s"(out.stride[0]), "s"(out.stride[1]), "s"(out.stride[2]),
               "s"(out.begin[1]), "s"(out.begin[2]));
  const int64_t n8 = N / 8;
  const int64_t total = T * n8;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / n8;
    const int32_t n = (int32_t)(i - t * n8) * 8;
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int32_t k0 = 0; k0 < nsplit; k0 += SB) {
      float4 a[SB], b[SB];
#pragma unroll
      for (int kk = 0; kk < SB; ++kk) {
        const int32_t k = min(k0 + kk, nsplit - 1);
        const float4* p = reinterpret_cast<const float4*>(part + ((int64_t)k * T + t) * N + n);
        a[kk] = p[0];
        b[kk] = p[1];
      }
#pragma unroll
      for (int kk = 0; kk < SB; ++kk) {
        if (k0 + kk < nsplit) {
          s[0] += a[kk].x; s[1] += a[kk].y; s[2] += a[kk].z; s[3] += a[kk].w;
          s[4] += b[kk].x; s[5] += b[kk].y; s[6] += b[kk].z; s[7] += b[kk].w;
        }
      }
    }
    const int sg = seg_of(out, n);
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = f2bf(s[e]);
    *reinterpret_cast<bf16x8*>(out.ptr[sg] + t * out.stride[sg] + (n - out.begin[sg])) = o;
  }
}

// Context K/V rows (the stacked [K | V] product of a propose step's appended
// rows): the K-slice partials summed in slice order and rounded to bf16, as
// split_sum_kernel stores them, and for the K heads then the per-head k-norm
// (RMSNorm over the 128 dims) and NeoX RoPE at the row's position, as
// qk_norm_rope_kernel applies them to those stored values; one launch instead
// of two. One head vector per 16 lanes: lane s holds dims [4s, 4s + 4) and
// their rotation partners [64 + 4s, 64 + 4s + 4).
constexpr int KR_DH = 128;
__global__ __launch_bounds__(256) void split_sum_krope_kernel(
    const float* __restrict__ part, int32_t nsplit, int64_t T, int32_t hkv, bf16* __restrict__ k_out,
    bf16* __restrict__ v_out, const float* __restrict__ knw, const int32_t* __restrict__ pos,
    const float2* __restrict__ table, int32_t max_pos, float eps) {
  // every argument in one batch of scalar loads (no dependent argument reads)
  asm volatile("" ::"s"(part), "s"(nsplit), "s"(T), "s"(hkv), "s"(k_out), "s"(v_out), "s"(knw),
               "s"(pos), "s"(table), "s"(max_pos), "s"(eps));
  constexpr int LANES = KR_DH / 8;
  constexpr int HALF = KR_DH / 2;
  const int s = (threadIdx.x & 63) % LANES;
  const int64_t vec = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LANES;  // 256-thread blocks
  const int32_t heads = 2 * hkv;
  const int32_t N = heads * KR_DH;
  const bool valid = vec < T * heads;  // shared by the 16 lanes of a vector
  const int64_t t = valid ? vec / heads : 0;
  const int32_t h = valid ? (int32_t)(vec % heads) : 0;
  const bool is_k = h < hkv;
  // The K heads' operands (position, then its cos/sin, and the k-norm
  // weights) are loaded ahead of the partials, so that their round trips
  // overlap the partials' instead of following them.
  float4 c01 = make_float4(0.f, 0.f, 0.f, 0.f), c23 = c01, w0 = c01, w1 = c01;
  if (valid && is_k) {
    int32_t p = pos[t];
    p = p < 0 ? 0 : (p >= max_pos ? max_pos - 1 : p);
    const float4* cs4 = reinterpret_cast<const float4*>(table + (int64_t)p * HALF + 4 * s);
    c01 = cs4[0];
    c23 = cs4[1];
    w0 = *reinterpret_cast<const float4*>(knw + 4 * s);
    w1 = *reinterpret_cast<const float4*>(knw + HALF + 4 * s);
  }
  float x0[4] = {0.f, 0.f, 0.f, 0.f}, x1[4] = {0.f, 0.f, 0.f, 0.f};
  if (valid) {
    const int32_t c0 = h * KR_DH + 4 * s;
    for (int32_t k0 = 0; k0 < nsplit; k0 += SB) {
      f32x4 a[SB], b[SB];
#pragma unroll
      for (int kk = 0; kk < SB; ++kk) {
        const int32_t k = min(k0 + kk, nsplit - 1);
        const float* p = part + ((int64_t)k * T + t) * N + c0;
        a[kk] = *reinterpret_cast<const f32x4*>(p);
        b[kk] = *reinterpret_cast<const f32x4*>(p + HALF);
      }
#pragma unroll
      for (int kk = 0; kk < SB; ++kk) {
        if (k0 + kk < nsplit) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x0[e] += a[kk][e];
            x1[e] += b[kk][e];
          }
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x0[e] = bf2f(f2bf(x0[e]));
      x1[e] = bf2f(f2bf(x1[e]));
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) ss += x0[e] * x0[e] + x1[e] * x1[e];
  ss = group_sum<LANES>(ss);
  const float inv = 1.0f / sqrtf(ss * (1.0f / KR_DH) + eps);
  if (!valid) return;
  bf16x4 o0, o1;
  bf16* dst;
  if (!is_k) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o0[e] = f2bf(x0[e]);
      o1[e] = f2bf(x1[e]);
    }
    dst = v_out + (t * hkv + (h - hkv)) * KR_DH;
  } else {
    const float cs[8] = {c01.x, c01.y, c01.z, c01.w, c23.x, c23.y, c23.z, c23.w};
    const float wa[4] = {w0.x, w0.y, w0.z, w0.w}, wb[4] = {w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float av = x0[e] * inv * wa[e];
      const float bv = x1[e] * inv * wb[e];
      const float c = cs[2 * e], sn = cs[2 * e + 1];
      o0[e] = f2bf(av * c - bv * sn);
      o1[e] = f2bf(bv * c + av * sn);
    }
    dst = k_out + (t * hkv + h) * KR_DH;
  }
  *reinterpret_cast<bf16x4*>(dst + 4 * s) = o0;
  *reinterpret_cast<bf16x4*>(dst + HALF + 4 * s) = o1;
}

struct ProjPlan {
  int64_t mtiles;
  int32_t bn, ntiles, nsplit, ksteps;
  size_t part_bytes;
};

// Wide outputs (N a multiple of 128 with at least 16 column tiles) use the
// 128 x 128 tile, one workgroup per CU, when each workgroup then still gets a
// long K slice (>= 12 steps): K is cut into nsplit slices of whole GBK-steps
// (the last one may be shorter) so that the tiles make at most one round of
// the CUs. With short slices the per-workgroup start-up and the partial tiles
// (64 KB each) outweigh the smaller activation share (measured: o_proj of the
// Qwen3-8B shape, 8 slices of 8 steps, 13.8 us against 10.8 us with 128 x 64
// tiles). Otherwise 128 x 64 tiles with K split in powers of two (slices of
// at least 256) until the tiles cover the CUs.
ProjPlan plan_proj(int64_t T, int32_t N, int32_t K, int num_cus, bool allow_wide = true) {
  ProjPlan pl{};
  pl.mtiles = (T + GBM - 1) / GBM;
  const int32_t steps = K / GBK;
  int64_t ns = 1;
  if (allow_wide && N % 128 == 0 && N / 128 >= 16) {
    const int64_t tiles = pl.mtiles * (N / 128);
    ns = std::max<int64_t>(1, num_cus / std::max<int64_t>(1, tiles));
  }
  if (allow_wide && N % 128 == 0 && N / 128 >= 16 && steps / ns >= 12) {
    pl.bn = 128;
    pl.ntiles = N / 128;
    pl.ksteps = (int32_t)((steps + ns - 1) / ns);
    pl.nsplit = (steps + pl.ksteps - 1) / pl.ksteps;  // no empty slice
  } else {
    pl.bn = 64;
    pl.ntiles = N / 64;
    pl.nsplit = 1;
    const int64_t tiles = pl.mtiles * pl.ntiles;
    while (tiles * pl.nsplit < num_cus && K % (pl.nsplit * 2 * GBK) == 0 && K / (pl.nsplit * 2) >= 256)
      pl.nsplit *= 2;
    pl.ksteps = steps / pl.nsplit;
  }
  pl.part_bytes = pl.nsplit > 1 ? (size_t)pl.nsplit * (size_t)T * (size_t)N * sizeof(float) : 0;
  return pl;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The product's grid (checked by the callers before their first launch).
bool proj_grid_fits(const ProjPlan& pl) { return grid_fits(pl.mtiles * pl.ntiles * pl.nsplit); }

// W's rows [0, n1) are read from w and rows [n1, N) from w2 (w2 == nullptr: all
// from w); n1 must be a multiple of the tile width.
hipError_t launch_proj(const bf16* a, const bf16* w, int64_t T, int32_t N, int32_t K,
                       const ProjPlan& pl, float* part, const OutSegs& out, hipStream_t s,
                       const bf16* w2 = nullptr, int32_t n1 = 0, bool sum_slices = true) {
  // The LDS limit is a per-function setting: raised once per device, not per
  // launch (stream capture then sees only the launches).
  static std::once_flag once[64];
  int dev = 0;
  (void)hipGetDevice(&dev);
  std::call_once(once[dev & 63], [] {
    (void)hipFuncSetAttribute((const void*)proj_gemm_kernel<64>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)GemmShape<64>::LDS);
    (void)hipFuncSetAttribute((const void*)proj_gemm_kernel<128>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)GemmShape<128>::LDS);
  });
  GemmArgs g{};
  g.a = a; g.w = w; g.T = T; g.N = N; g.K = K;
  g.w2 = w2 ? w2 : w;
  g.n1 = w2 ? n1 : N;
  g.ksteps = pl.ksteps; g.nsplit = pl.nsplit; g.part = part; g.out = out;
  const int64_t blocks = pl.mtiles * pl.ntiles * pl.nsplit;
  if (!grid_fits(blocks)) return hipErrorInvalidConfiguration;
  if (pl.bn == 128)
    hipLaunchKernelGGL(proj_gemm_kernel<128>, dim3((unsigned)blocks), dim3(GNT), GemmShape<128>::LDS,
                       s, g);
  else
    hipLaunchKernelGGL(proj_gemm_kernel<64>, dim3((unsigned)blocks), dim3(GNT), GemmShape<64>::LDS,
                       s, g);
  if (pl.nsplit > 1 && sum_slices) {
    const int64_t items = T * (N / 8);
    const int64_t sblocks = std::min<int64_t>((items + 255) / 256, 4096);
    hipLaunchKernelGGL(split_sum_kernel, dim3((unsigned)sblocks), dim3(256), 0, s,
                       (const float*)part, pl.nsplit, T, N, out);
  }
  return hipGetLastError();
}

}  // namespace

size_t block_qkv_workspace_bytes(int64_t T, int32_t hidden, int32_t hq, int32_t hkv, int32_t dh,
                                 int num_cus) {
  const int32_t n = (hq + 2 * hkv) * dh;
  const ProjPlan pl = plan_proj(T, n, hidden, num_cus);
  return align256((size_t)T * hidden * sizeof(bf16)) + align256(pl.part_bytes);
}

hipError_t launch_block_qkv(const void* hidden, void* residual, const float* norm_w,
                            const void* w_qkv, int64_t T, int32_t hidden_size, int32_t hq,
                            int32_t hkv, int32_t dh, float eps, void* q, void* k, void* v,
                            void* ws, int num_cus, hipStream_t s) {
  if (T == 0) return hipSuccess;
  bf16* normed = (bf16*)ws;
  const int32_t n = (hq + 2 * hkv) * dh;
  const ProjPlan pl = plan_proj(T, n, hidden_size, num_cus);
  if (!proj_grid_fits(pl) || !grid_fits(T)) return hipErrorInvalidConfiguration;
  float* part = (float*)((char*)ws + align256((size_t)T * hidden_size * sizeof(bf16)));
  if (residual)
    hipLaunchKernelGGL(residual_norm_kernel<true>, dim3((unsigned)T), dim3(256), 0, s,
                       (const bf16*)hidden, (bf16*)residual, norm_w, normed, hidden_size, eps);
  else
    hipLaunchKernelGGL(residual_norm_kernel<false>, dim3((unsigned)T), dim3(256), 0, s,
                       (const bf16*)hidden, (bf16*)nullptr, norm_w, normed, hidden_size, eps);
  OutSegs out{};
  out.ptr[0] = (bf16*)q; out.ptr[1] = (bf16*)k; out.ptr[2] = (bf16*)v;
  out.stride[0] = (int64_t)hq * dh; out.stride[1] = (int64_t)hkv * dh; out.stride[2] = (int64_t)hkv * dh;
  out.begin[0] = 0; out.begin[1] = hq * dh; out.begin[2] = (hq + hkv) * dh; out.begin[3] = n;
  return launch_proj(normed, (const bf16*)w_qkv, T, n, hidden_size, pl, part, out, s);
}

size_t o_proj_workspace_bytes(int64_t T, int32_t hidden, int32_t in_dim, int num_cus) {
  return align256(plan_proj(T, hidden, in_dim, num_cus).part_bytes);
}

hipError_t launch_o_proj(const void* attn, const void* w_o, int64_t T, int32_t hidden,
                         int32_t in_dim, void* out, void* ws, int num_cus, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const ProjPlan pl = plan_proj(T, hidden, in_dim, num_cus);
  OutSegs o{};
  o.ptr[0] = o.ptr[1] = o.ptr[2] = (bf16*)out;
  o.stride[0] = o.stride[1] = o.stride[2] = hidden;
  o.begin[0] = 0; o.begin[1] = o.begin[2] = o.begin[3] = hidden;
  return launch_proj((const bf16*)attn, (const bf16*)w_o, T, hidden, in_dim, pl, (float*)ws, o, s);
}

namespace {
// f32 -> bf16 (round to nearest even), 8 elements a thread.
__global__ __launch_bounds__(256) void cast_bf16_kernel(const float* __restrict__ src,
                                                        bf16* __restrict__ dst, int64_t n8) {
  asm volatile("" ::"s"(src), "s"(dst), "s"(n8));  // one batch of argument loads
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * blockDim.x) {
    const float4 a = reinterpret_cast<const float4*>(src)[2 * i];
    const float4 b = reinterpret_cast<const float4*>(src)[2 * i + 1];
    bf16x8 o;
    o[0] = f2bf(a.x); o[1] = f2bf(a.y); o[2] = f2bf(a.z); o[3] = f2bf(a.w);
    o[4] = f2bf(b.x); o[5] = f2bf(b.y); o[6] = f2bf(b.z); o[7] = f2bf(b.w);
    reinterpret_cast<bf16x8*>(dst)[i] = o;
  }
}
}  // namespace

// Context K/V of a few rows (a propose step's appended rows): the hidden
// RMSNorm as its own pass (bf16 rows), the K and V products as one split-K
// projection GEMM over the stacked weights, then the per-head k-norm + RoPE in
// place on K. A 256-row
// tile of the large-row kernel would leave most CUs idle at these sizes.
size_t context_kv_rows_workspace_bytes(int64_t T, int32_t hidden, int32_t hkv, int32_t dh,
                                       int num_cus) {
  return align256((size_t)T * hidden * sizeof(bf16)) +
         align256(plan_proj(T, 2 * hkv * dh, hidden, num_cus, (hkv * dh) % 128 == 0).part_bytes);
}

hipError_t launch_context_kv_rows(const void* hidden, const float* hnw, const void* wk,
                                  const void* wv, const float* knw, const int32_t* pos, int64_t T,
                                  int32_t hidden_size, int32_t hkv, int32_t dh, float eps,
                                  const float* table, int32_t max_pos, void* k_out, void* v_out,
                                  void* ws, int num_cus, hipStream_t s) {
  if (T == 0) return hipSuccess;
  bf16* normed = (bf16*)ws;
  float* part = (float*)((char*)ws + align256((size_t)T * hidden_size * sizeof(bf16)));
  // K and V in one product over the stacked [W_k; W_v] (columns [0, Hkv Dh) to
  // k_out, the rest to v_out)
  const int32_t n = hkv * dh;
  // (a 128-wide tile must not straddle the two weights)
  const ProjPlan pl = plan_proj(T, 2 * n, hidden_size, num_cus, n % 128 == 0);
  if (!proj_grid_fits(pl) || !grid_fits(T)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(residual_norm_kernel<false>, dim3((unsigned)T), dim3(256), 0, s,
                     (const bf16*)hidden, (bf16*)nullptr, hnw, normed, hidden_size, eps);
  OutSegs o{};
  o.ptr[0] = (bf16*)k_out; o.ptr[1] = o.ptr[2] = (bf16*)v_out;
  o.stride[0] = o.stride[1] = o.stride[2] = n;
  o.begin[0] = 0; o.begin[1] = n; o.begin[2] = o.begin[3] = 2 * n;
  if (pl.nsplit > 1 && dh == KR_DH) {
    // the slice sum also applies the k-norm and RoPE to the K heads
    hipError_t e = launch_proj(normed, (const bf16*)wk, T, 2 * n, hidden_size, pl, part, o, s,
                               (const bf16*)wv, n, /*sum_slices=*/false);
    if (e != hipSuccess) return e;
    const int64_t threads = T * 2 * hkv * (KR_DH / 8);
    hipLaunchKernelGGL(split_sum_krope_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       s, (const float*)part, pl.nsplit, T, hkv, (bf16*)k_out, (bf16*)v_out, knw,
                       pos, reinterpret_cast<const float2*>(table), max_pos, eps);
    return hipGetLastError();
  }
  hipError_t e = launch_proj(normed, (const bf16*)wk, T, 2 * n, hidden_size, pl, part, o, s,
                             (const bf16*)wv, n);
  if (e != hipSuccess) return e;
  return launch_qk_norm_rope(DFLASH_BF16, nullptr, k_out, nullptr, knw, pos, T, 0, hkv, dh, eps,
                             table, max_pos, s);
}

size_t fc_combine_workspace_bytes(int64_t T, int32_t hidden, int32_t taps, int num_cus) {
  const int32_t k = hidden * taps;
  return align256((size_t)T * k * sizeof(bf16)) + align256(plan_proj(T, hidden, k, num_cus).part_bytes);
}

hipError_t launch_fc_combine(const float* aux, const void* w_fc, int64_t T, int32_t hidden,
                             int32_t taps, void* out, void* ws, int num_cus, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int32_t k = hidden * taps;
  bf16* a = (bf16*)ws;
  const int64_t n8 = T * k / 8;
  const ProjPlan pl = plan_proj(T, hidden, k, num_cus);
  if (!proj_grid_fits(pl)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(cast_bf16_kernel, dim3((unsigned)std::min<int64_t>((n8 + 255) / 256, 4096)),
                     dim3(256), 0, s, aux, a, n8);
  float* part = (float*)((char*)ws + align256((size_t)T * k * sizeof(bf16)));
  OutSegs o{};
  o.ptr[0] = o.ptr[1] = o.ptr[2] = (bf16*)out;
  o.stride[0] = o.stride[1] = o.stride[2] = hidden;
  o.begin[0] = 0; o.begin[1] = o.begin[2] = o.begin[3] = hidden;
  return launch_proj(a, (const bf16*)w_fc, T, hidden, k, pl, part, o, s);
}

}  // namespace dflash
