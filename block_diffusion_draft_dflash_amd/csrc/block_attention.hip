// DFlash block attention: each block of B query rows of a request attends over
// that request's context K/V rows followed by the block's own K/V rows.
//
// "qwen3_dflash.cpp" page: file header (bidirectional in-block attention on
// full-attention layers, causal + sliding window on SWA layers),
// ForwardWithCtxKVDev (the per-request [context; block] sequence, only block
// query rows kept, scale 1/sqrt(Dh)) and ForwardPagedBody (block queries over
// a separate context store, no materialised combined sequence). The reference
// materialises the combined sequence with index copies and computes (then
// discards) every context query row; here the kernel reads the two packed
// sources directly and computes block queries only.
//
// bf16 kernel (the hot path), one workgroup = 4 waves per work unit:
//   unit = (request r, 64-row query tile, key range of `chunk` keys) x kv-head g
//   query tile rows = the (G q-heads of kv-head g) x (block rows) pairs,
//   flattened; wave w owns rows 16w..16w+15 (for G = 4, B = 16: q-head 4g+w).
//   Per 64-key tile: K and V rows of head g are streamed HBM -> registers ->
//   LDS (16-byte loads, XOR-swizzled rows, double buffered); S^T = K Q^T and
//   O^T += V^T P^T run on v_mfma_f32_16x16x32_bf16; V^T operands come straight
//   from the row-major V tile with ds_read_b64_tr_b16. Softmax is online in
//   f32 (base-2 exponent, scale*log2(e) folded into one multiply); the four
//   lanes that share a query row reduce with permlane swaps.
//   A request whose key range spans several units writes f32 partials
//   (unnormalised O, running max, sum); the last unit to finish (integer
//   ticket per (request, query tile, kv-head)) merges them in split order, so
//   the result is deterministic.
#include "dflash_device.h"
#include "dflash_internal.h"

namespace dflash {
namespace {

constexpr int QROWS = 64;  // query rows per work unit
constexpr int KT = 64;     // keys per tile
constexpr int NT = 256;    // threads per workgroup
constexpr float LOG2E = 1.4426950408889634f;

struct AttnArgs {
  const int32_t* cu_ctx;
  const int32_t* cu_blk;
  const bf16* q;
  const bf16* kb;
  const bf16* vb;
  const bf16* kc;
  const bf16* vc;
  bf16* out;
  float* part_o;      // [units * hkv][QROWS][DH]
  float* part_ml;     // [units * hkv][QROWS][2]
  int32_t* counters;  // [R][qtiles][hkv]
  int64_t total_ctx, total_blk;
  int32_t num_reqs, hq, hkv, group, chunk, qtiles, max_blk;
  float scale_log2;
  int32_t causal, window;
};

struct Unit {
  int32_t r, qt, s, nsplit, first;  // first = global unit index of split 0 of this (r, qt)
  int32_t clen, blen, lo;
  int32_t ctx0, blk0;
};

__device__ __forceinline__ int32_t clamp_nonneg(int32_t x) { return x < 0 ? 0 : x; }

// Row ranges of request r, clamped into the buffers' extents so that
// inconsistent device metadata can never index outside them.
__device__ __forceinline__ void request_rows(const int32_t* cu_ctx, const int32_t* cu_blk,
                                             int32_t r, int64_t total_ctx, int64_t total_blk,
                                             int32_t* c0, int32_t* c1, int32_t* b0, int32_t* b1) {
  const int32_t tc = (int32_t)total_ctx, tb = (int32_t)total_blk;
  *c0 = min(max(cu_ctx[r], 0), tc);
  *c1 = min(max(cu_ctx[r + 1], *c0), tc);
  *b0 = min(max(cu_blk[r], 0), tb);
  *b1 = min(max(cu_blk[r + 1], *b0), tb);
}

// Lengths of request r and its unit count (0 if the request has no block rows).
__device__ __forceinline__ void request_shape(const AttnArgs& a, int32_t r, int32_t* clen,
                                              int32_t* blen, int32_t* lo, int32_t* ns,
                                              int32_t* nq) {
  int32_t c0, c1, b0, b1;
  request_rows(a.cu_ctx, a.cu_blk, r, a.total_ctx, a.total_blk, &c0, &c1, &b0, &b1);
  *clen = c1 - c0;
  *blen = min(b1 - b0, a.max_blk);
  *lo = (a.causal && a.window > 0) ? clamp_nonneg(*clen - a.window + 1) : 0;
  const int32_t n = *clen + *blen - *lo;
  *ns = *blen > 0 ? (n + a.chunk - 1) / a.chunk : 0;
  *nq = *blen > 0 ? (a.group * *blen + QROWS - 1) / QROWS : 0;
}

// Find work unit u by a wave-wide prefix scan over the requests' unit counts.
// Every wave of the workgroup computes the same answer from the same data.
__device__ bool find_unit(const AttnArgs& a, int32_t u, Unit* out) {
  const int lane = threadIdx.x & 63;
  int32_t base = 0;
  for (int32_t r0 = 0; r0 < a.num_reqs; r0 += 64) {
    const int32_t r = r0 + lane;
    int32_t cnt = 0;
    if (r < a.num_reqs) {
      int32_t cl, bl, lo, ns, nq;
      request_shape(a, r, &cl, &bl, &lo, &ns, &nq);
      cnt = ns * nq;
    }
    int32_t incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t t = __shfl_up(incl, off, 64);
      if (lane >= off) incl += t;
    }
    const int32_t total = __shfl(incl, 63, 64);
    if (u < base + total) {
      const unsigned long long hit = __ballot(base + incl > u);
      const int idx = __ffsll((long long)hit) - 1;
      const int32_t rr = r0 + idx;
      const int32_t start = base + __shfl(incl - cnt, idx, 64);
      int32_t cl, bl, lo, ns, nq;
      request_shape(a, rr, &cl, &bl, &lo, &ns, &nq);
      const int32_t loc = u - start;
      out->r = rr;
      out->qt = loc / ns;
      out->s = loc % ns;
      out->nsplit = ns;
      out->first = start + out->qt * ns;
      out->clen = cl;
      out->blen = bl;
      out->lo = lo;
      int32_t c0, c1, b0, b1;
      request_rows(a.cu_ctx, a.cu_blk, rr, a.total_ctx, a.total_blk, &c0, &c1, &b0, &b1);
      out->ctx0 = c0;
      out->blk0 = b0;
      return true;
    }
    base += total;
  }
  return false;
}

// Physical 16-byte chunk of logical chunk c in LDS row `row` (bank spreading).
template <int DH>
__device__ __forceinline__ int swz(int row, int c) {
  if constexpr (DH == 128) return c ^ (row & 15);
  else return c ^ ((row >> 1) & 7);
}

template <int DH>
__global__ __launch_bounds__(NT) void block_attn_bf16_kernel(AttnArgs a) {
  constexpr int CH = DH / 8;             // 16-byte chunks per row
  constexpr int DS = DH / 32;            // MFMA k-steps over the head dim
  constexpr int DT = DH / 16;            // 16-wide d tiles of O^T
  constexpr int LOADS = KT * CH / NT;    // 16-byte loads per thread per tensor per tile
  constexpr int TILE_ELEMS = KT * DH;
  extern __shared__ __attribute__((aligned(16))) bf16 smem[];  // [stage][K|V][KT*DH]

  const int32_t g = blockIdx.x % a.hkv;
  const int32_t u = blockIdx.x / a.hkv;
  Unit un;
  if (!find_unit(a, u, &un)) return;  // uniform over the workgroup

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int m = lane & 15;   // query row within the wave / MFMA column
  const int j = lane >> 4;   // lane group

  const int32_t n_all = un.clen + un.blen;
  const int32_t k_begin = un.lo + un.s * a.chunk;
  const int32_t k_end = min(k_begin + a.chunk, n_all);
  const int32_t ntiles = (k_end - k_begin + KT - 1) / KT;

  // This lane's query row.
  const int32_t nrows = a.group * un.blen;
  const int32_t nq = un.qt * QROWS + 16 * w + m;
  const int32_t hl = nq / un.blen;
  const int32_t b = nq - hl * un.blen;
  const int64_t qrow = (int64_t)un.blk0 + b;
  const bool rvalid = nq < nrows && qrow < a.total_blk;
  const int32_t qhead = g * a.group + hl;
  const int32_t qidx = un.clen + b;  // index of this query in [context; block]

  bf16x8 qf[DS];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) {
    if (rvalid)
      qf[ds] = *reinterpret_cast<const bf16x8*>(a.q + (qrow * a.hq + qhead) * DH + (j + 4 * ds) * 8);
    else
      qf[ds] = bf16x8{};
  }

  // Tile loader: thread tid moves chunks tid, tid+256, ... of the K and V tiles.
  bf16x8 kreg[LOADS], vreg[LOADS];
  auto load_tile = [&](int32_t kt0) {
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int id = tid + NT * it;
      const int kk = id / CH;
      const int c = id % CH;
      const int32_t kidx = kt0 + kk;
      const bf16* ks = nullptr;
      const bf16* vs = nullptr;
      if (kidx < k_end) {
        if (kidx < un.clen) {
          const int64_t row = (int64_t)un.ctx0 + kidx;
          if (row < a.total_ctx) {
            const int64_t off = (row * a.hkv + g) * DH + c * 8;
            ks = a.kc + off;
            vs = a.vc + off;
          }
        } else {
          const int64_t row = (int64_t)un.blk0 + (kidx - un.clen);
          if (row < a.total_blk) {
            const int64_t off = (row * a.hkv + g) * DH + c * 8;
            ks = a.kb + off;
            vs = a.vb + off;
          }
        }
      }
      kreg[it] = ks ? *reinterpret_cast<const bf16x8*>(ks) : bf16x8{};
      vreg[it] = vs ? *reinterpret_cast<const bf16x8*>(vs) : bf16x8{};
    }
  };
  auto store_tile = [&](int st) {
    bf16* kd = smem + st * 2 * TILE_ELEMS;
    bf16* vd = kd + TILE_ELEMS;
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int id = tid + NT * it;
      const int kk = id / CH;
      const int c = id % CH;
      const int off = kk * DH + swz<DH>(kk, c) * 8;
      *reinterpret_cast<bf16x8*>(kd + off) = kreg[it];
      *reinterpret_cast<bf16x8*>(vd + off) = vreg[it];
    }
  };

  f32x4 acc_o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc_o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mx = -INFINITY;  // running max (log2 domain) of this lane's query row
  float lsum = 0.f;      // this lane's share of the running sum

  // Masking is needed on tiles with keys past the range end, or that reach
  // beyond the first query (causal) or before the last query's window.
  const int32_t qmin = un.clen;                 // smallest query index
  const int32_t qmax = un.clen + un.blen - 1;   // largest query index

  load_tile(k_begin);
  store_tile(0);
  __syncthreads();

  for (int32_t it = 0; it < ntiles; ++it) {
    const int st = it & 1;
    const int32_t kt0 = k_begin + it * KT;
    const bool has_next = it + 1 < ntiles;
    if (has_next) load_tile(kt0 + KT);

    const bf16* kd = smem + st * 2 * TILE_ELEMS;
    const bf16* vd = kd + TILE_ELEMS;

    // S^T = K Q^T for the 4 sub-tiles of 16 keys.
    f32x4 sacc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int row = 16 * t + m;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        const bf16x8 kf =
            *reinterpret_cast<const bf16x8*>(kd + row * DH + swz<DH>(row, j + 4 * ds) * 8);
        sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ds], sacc[t], 0, 0, 0);
      }
    }

    // Online softmax on this lane's 16 keys (16t + 4j + i) of query row m.
    const bool need_mask = (kt0 + KT > k_end) ||
                           (a.causal && (kt0 + KT - 1 > qmin ||
                                         (a.window > 0 && kt0 <= qmax - a.window)));
    float sv[4][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = sacc[t][i] * a.scale_log2;
        if (need_mask) {
          const int32_t kidx = kt0 + 16 * t + 4 * j + i;
          bool vis = kidx < k_end;
          if (a.causal) {
            vis = vis && kidx <= qidx;
            if (a.window > 0) vis = vis && (qidx - kidx) < a.window;
          }
          v = vis ? v : -INFINITY;
        }
        sv[t][i] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = xrow4_max(tmax);
    const float mnew = fmaxf(mx, tmax);
    const float msafe = (mnew == -INFINITY) ? 0.f : mnew;
    const float alpha = fast_exp2(mx - msafe);
    mx = mnew;
    float psum = 0.f;
    bf16x8 pf[2];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = fast_exp2(sv[t][i] - msafe);
        psum += p;
        pf[t >> 1][(t & 1) * 4 + i] = f2bf(p);
      }
    lsum = lsum * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc_o[dt] = acc_o[dt] * alpha;

    // O^T += V^T P^T over two 32-key steps. The transpose read hands lane i of
    // group j the column (16dt + i) of rows key(j, e); source lane s supplies
    // row 32ks + 16h + 4j + s/4, columns 16dt + 4(s%4) .. +3.
    const int src_row = 4 * j + (m >> 2);
    const int src_col4 = (m & 3) * 4;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        bf16x8 vf;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int row = 32 * ks + 16 * h + src_row;
          const int col = 16 * dt + src_col4;
          const int off = row * DH + swz<DH>(row, col >> 3) * 8 + (col & 7);
          const i16x4 tv = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (DF_LDS i16x4*)((DF_LDS bf16*)(vd + off)));
          const bf16x4 bv = __builtin_bit_cast(bf16x4, tv);
#pragma unroll
          for (int e = 0; e < 4; ++e) vf[4 * h + e] = bv[e];
        }
        acc_o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[ks], acc_o[dt], 0, 0, 0);
      }
    }

    if (has_next) store_tile(st ^ 1);
    __syncthreads();
  }

  const float ltot = xrow4_sum(lsum);
  const int32_t nrow_unit = 16 * w + m;  // row within the unit's query tile

  if (un.nsplit == 1) {
    if (rvalid) {
      const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
      bf16* dst = a.out + (qrow * a.hq + qhead) * DH + 4 * j;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        bf16x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = f2bf(acc_o[dt][i] * inv);
        *reinterpret_cast<bf16x4*>(dst + 16 * dt) = o;
      }
    }
    return;
  }

  // Split: publish the partial, then the last unit of (r, qt, g) merges.
  {
    float* po = a.part_o + ((int64_t)blockIdx.x * QROWS + nrow_unit) * DH + 4 * j;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<f32x4*>(po + 16 * dt) = acc_o[dt];
    if (j == 0) {
      float2* pml = reinterpret_cast<float2*>(a.part_ml) + (int64_t)blockIdx.x * QROWS + nrow_unit;
      *pml = make_float2(mx, ltot);
    }
  }
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  int32_t* ctr = a.counters + ((int64_t)un.r * a.qtiles + un.qt) * a.hkv + g;
  if (tid == 0) s_last = (atomicAdd(ctr, 1) == un.nsplit - 1);
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // Merge: thread -> (row, quarter of the head dim); splits in index order.
  const int row = tid >> 2;
  const int dq = (tid & 3) * (DH / 4);
  const int32_t nq2 = un.qt * QROWS + row;
  float mmax = -INFINITY;
  for (int32_t s = 0; s < un.nsplit; ++s) {
    const int64_t slot = (int64_t)(un.first + s) * a.hkv + g;
    const float2 ml = reinterpret_cast<const float2*>(a.part_ml)[slot * QROWS + row];
    mmax = fmaxf(mmax, ml.x);
  }
  const float msafe = (mmax == -INFINITY) ? 0.f : mmax;
  float o[DH / 4];
#pragma unroll
  for (int d = 0; d < DH / 4; ++d) o[d] = 0.f;
  float L = 0.f;
  for (int32_t s = 0; s < un.nsplit; ++s) {
    const int64_t slot = (int64_t)(un.first + s) * a.hkv + g;
    const float2 ml = reinterpret_cast<const float2*>(a.part_ml)[slot * QROWS + row];
    const float wgt = fast_exp2(ml.x - msafe);
    L += ml.y * wgt;
    const float* src = a.part_o + (slot * QROWS + row) * DH + dq;
#pragma unroll
    for (int d = 0; d < DH / 4; d += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(src + d);
      o[d] += v[0] * wgt;
      o[d + 1] += v[1] * wgt;
      o[d + 2] += v[2] * wgt;
      o[d + 3] += v[3] * wgt;
    }
  }
  if (nq2 < nrows) {
    const int32_t hl2 = nq2 / un.blen;
    const int32_t b2 = nq2 - hl2 * un.blen;
    const int64_t qrow2 = (int64_t)un.blk0 + b2;
    if (qrow2 < a.total_blk) {
      const float inv = L > 0.f ? 1.0f / L : 0.f;
      bf16* dst = a.out + (qrow2 * a.hq + g * a.group + hl2) * DH + dq;
#pragma unroll
      for (int d = 0; d < DH / 4; d += 8) {
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = f2bf(o[d + e] * inv);
        *reinterpret_cast<bf16x8*>(dst + d) = v;
      }
    }
  }
  if (tid == 0) *ctr = 0;  // leave the ticket zeroed for the next call
}

// ----------------------------------------------------------------------------
// f32 kernel: one wave per (block row, q-head), exact-order f32 arithmetic.
// Lane <-> key for the scores, lane <-> head-dim slice for the output.
struct F32Args {
  const int32_t* cu_ctx;
  const int32_t* cu_blk;
  const float* q;
  const float* kb;
  const float* vb;
  const float* kc;
  const float* vc;
  float* out;
  int64_t total_ctx, total_blk;
  int32_t num_reqs, hq, hkv, group;
  float scale;
  int32_t causal, window;
};

template <int DH>
__global__ __launch_bounds__(64) void block_attn_f32_kernel(F32Args a) {
  constexpr int PER = DH / 64;
  const int lane = threadIdx.x;
  const int64_t t = blockIdx.x / a.hq;
  const int32_t h = blockIdx.x % a.hq;
  const int32_t g = h / a.group;
  // request owning block row t: last r with cu_blk[r] <= t
  int32_t lo = 0, hi = a.num_reqs - 1;
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if (a.cu_blk[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int32_t r = lo;
  int32_t c0, c1, b0, b1;
  request_rows(a.cu_ctx, a.cu_blk, r, a.total_ctx, a.total_blk, &c0, &c1, &b0, &b1);
  const int32_t clen = c1 - c0;
  const int32_t blen = b1 - b0;
  const int32_t b = (int32_t)(t - b0);
  if (b < 0 || b >= blen) return;
  const int32_t qidx = clen + b;
  const int32_t n = clen + blen;

  float qv[DH];
  const float* qp = a.q + (t * a.hq + h) * DH;
#pragma unroll
  for (int d = 0; d < DH; d += 4) {
    const float4 v = *reinterpret_cast<const float4*>(qp + d);
    qv[d] = v.x; qv[d + 1] = v.y; qv[d + 2] = v.z; qv[d + 3] = v.w;
  }
  float o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.f;
  float mx = -INFINITY, lpart = 0.f;
  for (int32_t k0 = 0; k0 < n; k0 += 64) {
    const int32_t kidx = k0 + lane;
    bool vis = kidx < n;
    if (a.causal) {
      vis = vis && kidx <= qidx;
      if (a.window > 0) vis = vis && (qidx - kidx) < a.window;
    }
    const float* krow = nullptr;
    const float* vrow_mine = nullptr;
    if (vis) {
      if (kidx < clen) {
        const int64_t row = (int64_t)c0 + kidx;
        if (row < a.total_ctx) { krow = a.kc + (row * a.hkv + g) * DH; vrow_mine = a.vc + (row * a.hkv + g) * DH; }
      } else {
        const int64_t row = (int64_t)b0 + (kidx - clen);
        if (row < a.total_blk) { krow = a.kb + (row * a.hkv + g) * DH; vrow_mine = a.vb + (row * a.hkv + g) * DH; }
      }
    }
    float s = -INFINITY;
    if (krow) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < DH; d += 4) {
        const float4 v = *reinterpret_cast<const float4*>(krow + d);
        acc += qv[d] * v.x + qv[d + 1] * v.y + qv[d + 2] * v.z + qv[d + 3] * v.w;
      }
      s = acc * a.scale;
    }
    float cmax = s;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) cmax = fmaxf(cmax, __shfl_xor(cmax, off, 64));
    const float mnew = fmaxf(mx, cmax);
    const float msafe = (mnew == -INFINITY) ? 0.f : mnew;
    const float alpha = expf(mx - msafe);
    mx = mnew;
    const float p = krow ? expf(s - msafe) : 0.f;
    lpart = lpart * alpha + p;
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] *= alpha;
    const uint64_t vaddr = (uint64_t)vrow_mine;
    for (int kk = 0; kk < 64; ++kk) {
      const float pk = __shfl(p, kk, 64);
      if (pk != 0.f) {
        const float* vr = (const float*)__shfl((long long)vaddr, kk, 64);
#pragma unroll
        for (int e = 0; e < PER; ++e) o[e] += pk * vr[lane + 64 * e];
      }
    }
  }
  float l = lpart;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off, 64);
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  float* op = a.out + (t * a.hq + h) * DH;
#pragma unroll
  for (int e = 0; e < PER; ++e) op[lane + 64 * e] = o[e] * inv;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace

bool plan_block_attention(const dflash_block_attn_params& p, int num_cus, AttnPlan* plan) {
  AttnPlan pl{};
  pl.group = p.num_q_heads / p.num_kv_heads;
  const int64_t qt = ((int64_t)pl.group * p.max_blk_len + QROWS - 1) / QROWS;
  pl.qtiles = (int32_t)(qt < 1 ? 1 : qt);
  int64_t eff = p.total_ctx + p.total_blk;
  if (p.causal && p.window > 0) {
    const int64_t bound = (int64_t)p.num_reqs * (p.window - 1) + p.total_blk;
    if (bound < eff) eff = bound;
  }
  if (p.split_keys > 0) {
    pl.chunk = p.split_keys;
  } else {
    const int64_t target = 2LL * (num_cus > 0 ? num_cus : 256);
    const int64_t work = eff * p.num_kv_heads * pl.qtiles;
    int64_t c = (work + target - 1) / target;
    c = (c + KT - 1) / KT * KT;
    if (c < 128) c = 128;
    if (c > (1 << 20)) c = 1 << 20;
    pl.chunk = (int32_t)c;
  }
  pl.units = (int64_t)pl.qtiles * ((eff + pl.chunk - 1) / pl.chunk + p.num_reqs);
  size_t off = 256;  // reserved header
  pl.off_counters = off;
  off = align_up(off + sizeof(int32_t) * (size_t)p.num_reqs * pl.qtiles * p.num_kv_heads, 256);
  pl.off_part_o = off;
  off = align_up(off + sizeof(float) * (size_t)pl.units * p.num_kv_heads * QROWS * p.head_dim, 256);
  pl.off_part_ml = off;
  off = align_up(off + sizeof(float) * 2 * (size_t)pl.units * p.num_kv_heads * QROWS, 256);
  pl.bytes = (p.dtype == DFLASH_BF16) ? off : 0;
  *plan = pl;
  return true;
}

hipError_t launch_block_attention(const dflash_block_attn_params& p, const AttnPlan& plan,
                                  const int32_t* cu_ctx, const int32_t* cu_blk, const void* q,
                                  const void* kb, const void* vb, const void* kc, const void* vc,
                                  void* out, void* ws, hipStream_t s) {
  if (p.dtype == DFLASH_F32) {
    F32Args a{};
    a.cu_ctx = cu_ctx; a.cu_blk = cu_blk;
    a.q = (const float*)q; a.kb = (const float*)kb; a.vb = (const float*)vb;
    a.kc = (const float*)kc; a.vc = (const float*)vc; a.out = (float*)out;
    a.total_ctx = p.total_ctx; a.total_blk = p.total_blk;
    a.num_reqs = p.num_reqs; a.hq = p.num_q_heads; a.hkv = p.num_kv_heads;
    a.group = plan.group; a.scale = p.scale; a.causal = p.causal ? 1 : 0; a.window = p.window;
    const int64_t blocks = p.total_blk * p.num_q_heads;
    if (p.head_dim == 128)
      hipLaunchKernelGGL(block_attn_f32_kernel<128>, dim3((unsigned)blocks), dim3(64), 0, s, a);
    else
      hipLaunchKernelGGL(block_attn_f32_kernel<64>, dim3((unsigned)blocks), dim3(64), 0, s, a);
    return hipGetLastError();
  }
  AttnArgs a{};
  a.cu_ctx = cu_ctx; a.cu_blk = cu_blk;
  a.q = (const bf16*)q; a.kb = (const bf16*)kb; a.vb = (const bf16*)vb;
  a.kc = (const bf16*)kc; a.vc = (const bf16*)vc; a.out = (bf16*)out;
  char* w = (char*)ws;
  a.counters = (int32_t*)(w + plan.off_counters);
  a.part_o = (float*)(w + plan.off_part_o);
  a.part_ml = (float*)(w + plan.off_part_ml);
  a.total_ctx = p.total_ctx; a.total_blk = p.total_blk;
  a.num_reqs = p.num_reqs; a.hq = p.num_q_heads; a.hkv = p.num_kv_heads;
  a.group = plan.group; a.chunk = plan.chunk; a.qtiles = plan.qtiles;
  a.max_blk = p.max_blk_len;
  a.scale_log2 = p.scale * LOG2E;
  a.causal = p.causal ? 1 : 0; a.window = p.window;
  const int64_t blocks = plan.units * p.num_kv_heads;
  const size_t lds = 2 * 2 * (size_t)KT * p.head_dim * sizeof(bf16);
  if (p.head_dim == 128) {
    hipFuncSetAttribute((const void*)block_attn_bf16_kernel<128>,
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(block_attn_bf16_kernel<128>, dim3((unsigned)blocks), dim3(NT), lds, s, a);
  } else {
    hipFuncSetAttribute((const void*)block_attn_bf16_kernel<64>,
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(block_attn_bf16_kernel<64>, dim3((unsigned)blocks), dim3(NT), lds, s, a);
  }
  return hipGetLastError();
}

}  // namespace dflash
