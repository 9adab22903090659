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
//   unit = (request r, 64-row query tile, range of keys) x kv-head g
//   query tile rows = the (G q-heads of kv-head g) x (block rows) pairs,
//   flattened; wave w owns rows 16w..16w+15 (for G = 4, B = 16: q-head 4g+w).
//   Each request's visible keys are cut into equal splits (whole tiles),
//   sized so that the units fill the machine; the plan is made on the host
//   when host copies of the lengths are given, else by every workgroup from
//   the device lengths. Per 32-key tile, the K and V rows of head g are
//   copied HBM -> LDS directly (16-byte lanes, XOR-swizzled rows, NSTAGE
//   stages, explicit waits); S^T = K Q^T and O^T += V^T P^T run on
//   v_mfma_f32_16x16x32_bf16, the V^T operands read from the row-major V tile
//   with ds_read_b64_tr_b16. Softmax is online in f32 (base-2 exponent,
//   scale*log2(e) folded into one multiply, rescale only when a row max grows
//   past a threshold); the four lanes that share a query row reduce with
//   permlane swaps. With the fused prologue the raw q rows are normed and
//   rotated in registers and the block's K rows in LDS.
//   A unit of a split request writes its partial (O / l scaled by a per-row
//   power of two into fp16, with max, sum and the scale's exponent in f32); a
//   second kernel merges each request's splits in split order, so the result
//   is deterministic.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "dflash_device.h"
#include "dflash_internal.h"

namespace dflash {
namespace {

constexpr int QROWS = 64;  // query rows per work unit
constexpr int PAGE = 16;   // rows per page of the paged context store
constexpr int PAGED_MAX_UNIT_KEYS = 16384;             // keys per unit over a paged store
constexpr int PG_MAX = PAGED_MAX_UNIT_KEYS / PAGE + 64;  // page ids a unit stages in LDS
constexpr int POS_LDS = 4 * 64;  // block positions staged by the fused prologue (64 per wave)
constexpr int KT = 32;     // keys per tile
constexpr int NT = 256;    // threads per workgroup
constexpr float LOG2E = 1.4426950408889634f;

// Phase trace (diagnostic build, -DDFLASH_PHASE_TRACE, libdflash_phasetrace.so):
// every workgroup of both kernels writes one record of 8 u64 to a region at
// the end of the workspace: the 100 MHz real-time counter at its start, after
// the unit lookup, at the loop's start and end and at its end, its XCD, its
// tile count and its kind (1: main kernel, 2: merge kernel). The product
// build compiles none of it.
#ifdef DFLASH_PHASE_TRACE
constexpr bool kPhaseTrace = true;
#else
constexpr bool kPhaseTrace = false;
#endif
__device__ __forceinline__ uint64_t pt_now() {
  if constexpr (kPhaseTrace) return __builtin_amdgcn_s_memrealtime();
  return 0;
}
__device__ __forceinline__ void pt_record(uint64_t* rec, uint64_t t0, uint64_t t1, uint64_t t2,
                                          uint64_t t3, int64_t tiles, int kind) {
  if constexpr (kPhaseTrace) {
    if (threadIdx.x == 0) {
      uint32_t xcc;
      asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
      const uint64_t t4 = __builtin_amdgcn_s_memrealtime();
      rec[0] = t0; rec[1] = t1; rec[2] = t2; rec[3] = t3; rec[4] = t4;
      rec[5] = xcc; rec[6] = (uint64_t)tiles; rec[7] = (uint64_t)kind;
    }
  }
}

// Work split planned on the host from host copies of the lengths, passed
// by value with the launch (kernel arguments): for each request its rows,
// visible key range, split size, split count and first unit, and the launch
// order of the units (per kv-head) as (request, index within the request's
// units), largest units first so that the dispatcher's in-order list
// scheduling balances unequal units. A unit's partial slot is its canonical
// (request-major) index, whatever its launch position. nreq == 0: plan on the
// device instead.
constexpr int HS_MAX_REQS = 64;
constexpr int HS_MAX_UNITS = 512;
struct ReqSched {
  int32_t c0, b0, clen, blen, lo, csz, ns, ubase;
};
struct HostSched {
  int32_t nreq, chunk, nunits, pad;
  uint16_t order[HS_MAX_UNITS];  // launch position -> (request << 8) | unit index in request
  ReqSched req[HS_MAX_REQS];
};

struct AttnArgs {
  const int32_t* cu_ctx;
  const int32_t* cu_blk;
  const bf16* q;
  const bf16* kb;
  const bf16* vb;
  const bf16* kc;
  const bf16* vc;
  bf16* out;
  f16* part_o;        // [units * hkv][QROWS][DH]: O / l of each split times 2^-e (fp16)
  float* part_ml;     // [units * hkv][QROWS][4]: max, sum, e, 0
  int32_t* dir;       // [R][qtiles][hkv]: first unit index of each split set
  int64_t total_ctx, total_blk;
  int32_t* hdr;       // workspace header: [0] = keys per split chosen for this call
  // the merge kernel reads hkv .. hplan together (one scalar load)
  int32_t hq, hkv, group, qtiles, num_reqs;
  int32_t hplan;      // = hs.nreq
  int32_t max_blk;
  int32_t chunk;      // keys per split (multiple of KT), or 0: chosen on the device
  int32_t units;      // work units per kv-head in the grid (grid = units * hkv)
  int32_t units_pref; // unit budget tried first (the packed call's; <= units)
  // Paged context store (bt == nullptr: packed context rows).
  const int32_t* bt;  // [num_reqs][bt_stride] page ids
  int32_t bt_stride;
  int32_t num_pages_m1;  // num_pages - 1 (clamped to int32)
  // Fused q/k prologue (q and k_blk raw): per-head RMSNorm + NeoX RoPE.
  const float* qnw;     // [Dh]
  const float* knw;     // [Dh]
  const int32_t* bpos;  // [total_blk] positions of the block rows
  const float2* rope;   // [max_pos][Dh/2] (cos, sin)
  int32_t max_pos;
  float eps;
  float scale_log2;
  int32_t causal, window;
  uint64_t* trace;     // phase-trace records (diagnostic build), else unused
  int64_t trace_main;  // records of the main kernel (the merge kernel's follow)
  HostSched hs;
};

struct Unit {
  int32_t r, qt, s, nsplit, first;  // first = global unit index of split 0 of this (r, qt)
  int32_t clen, blen, lo, csz;      // csz = keys per split of this request
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

// Lengths of one request as a lane holds them: first rows, context and block
// lengths, first visible key, number of visible keys, query tiles.
struct LaneReq {
  int32_t c0, b0, clen, blen, lo, n, nq;
};
__device__ __forceinline__ LaneReq lane_req(const AttnArgs& a, int32_t r) {
  LaneReq q{};
  if (r >= a.num_reqs) return q;
  int32_t c1, b1;
  request_rows(a.cu_ctx, a.cu_blk, r, a.total_ctx, a.total_blk, &q.c0, &c1, &q.b0, &b1);
  q.clen = c1 - q.c0;
  q.blen = min(b1 - q.b0, a.max_blk);
  q.lo = (a.causal && a.window > 0) ? clamp_nonneg(q.clen - a.window + 1) : 0;
  q.n = q.blen > 0 ? q.clen + q.blen - q.lo : 0;
  q.nq = q.blen > 0 ? (a.group * q.blen + QROWS - 1) / QROWS : 0;
  return q;
}
// The key range [lo, clen + blen) of a request is cut into ns = ceil(n / chunk)
// splits of equal size csz (rounded up to whole tiles); since chunk is a
// multiple of the tile, the last split is never empty.
__device__ __forceinline__ int32_t req_splits(const LaneReq& q, int32_t chunk) {
  return q.n > 0 ? (q.n + chunk - 1) / chunk : 0;
}
__device__ __forceinline__ int32_t req_split_size(const LaneReq& q, int32_t ns) {
  return ns > 0 ? ((q.n + ns - 1) / ns + KT - 1) / KT * KT : 0;
}

__device__ __forceinline__ int64_t wave_sum64(int64_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ int32_t wave_max(int32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off, 64));
  return v;
}

// The requests, 64 per lane group. Up to 64 requests they are loaded once and
// kept in registers; beyond that each group is re-read when needed.
struct ReqView {
  const AttnArgs& a;
  LaneReq cached;
  __device__ ReqView(const AttnArgs& args) : a(args) {
    cached = lane_req(a, threadIdx.x & 63);
  }
  __device__ __forceinline__ LaneReq group(int32_t r0) const {
    return r0 == 0 ? cached : lane_req(a, r0 + (threadIdx.x & 63));
  }
};

// Keys per split for this call. With a fixed split size requested, that one;
// otherwise the smallest multiple of KT whose total unit count fits the
// launched grid (a.units per kv-head), so that the grid is one balanced round
// of equal-sized units. Every workgroup computes the same value from the same
// lengths. The host guarantees a.units >= sum of nq_r, i.e. one unit per
// (request, query tile) always fits.
__device__ int32_t choose_chunk_for(const AttnArgs& a, const ReqView& rv, int32_t units);
// Over a paged store a unit spans at most PAGED_MAX_UNIT_KEYS keys (its page
// ids are staged in LDS): the packed call's budget is tried first, so the two
// calls split alike whenever that fits.
__device__ int32_t choose_chunk(const AttnArgs& a, const ReqView& rv) {
  if (a.chunk > 0) return a.chunk;
  const int32_t c = choose_chunk_for(a, rv, a.units_pref);
  if (a.bt == nullptr || c <= PAGED_MAX_UNIT_KEYS || a.units_pref >= a.units) return c;
  return choose_chunk_for(a, rv, a.units);
}
__device__ int32_t choose_chunk_for(const AttnArgs& a, const ReqView& rv, int32_t units) {
  auto count = [&](int32_t c) {
    int64_t tot = 0;
    for (int32_t r0 = 0; r0 < a.num_reqs; r0 += 64) {
      const LaneReq q = rv.group(r0);
      tot += wave_sum64((int64_t)req_splits(q, c) * q.nq);
    }
    return tot;
  };
  int32_t maxn = 0;
  int64_t work = 0;
  for (int32_t r0 = 0; r0 < a.num_reqs; r0 += 64) {
    const LaneReq q = rv.group(r0);
    maxn = max(maxn, wave_max(q.n));
    work += wave_sum64((int64_t)((q.n + KT - 1) / KT) * q.nq);  // in tiles
  }
  const int32_t kmax = max(1, (maxn + KT - 1) / KT);
  int32_t klo = (int32_t)max((int64_t)1, min((int64_t)kmax, (work + units - 1) / max(units, 1)));
  if (count(klo * KT) <= units) return klo * KT;
  // grow geometrically, then bisect: count() is non-increasing in c
  int32_t khi = klo, step = 1;
  while (khi < kmax) {
    khi = min(kmax, khi + step);
    step *= 2;
    if (count(khi * KT) <= units) break;
    klo = khi;
  }
  while (khi - klo > 1) {
    const int32_t mid = (klo + khi) / 2;
    if (count(mid * KT) <= units) khi = mid; else klo = mid;
  }
  return khi * KT;
}

// Find work unit u (for split size `chunk`) by a wave-wide prefix scan over
// the requests' unit counts; the owning lane's values are read back with
// readlane. Every wave of the workgroup computes the same answer.
__device__ bool find_unit(const AttnArgs& a, const ReqView& rv, int32_t chunk, int32_t u,
                          Unit* out) {
  const int lane = threadIdx.x & 63;
  int32_t base = 0;
  for (int32_t r0 = 0; r0 < a.num_reqs; r0 += 64) {
    const LaneReq q = rv.group(r0);
    const int32_t ns = req_splits(q, chunk);
    const int32_t cnt = ns * q.nq;
    int32_t incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t t = __shfl_up(incl, off, 64);
      if (lane >= off) incl += t;
    }
    const int32_t total = __builtin_amdgcn_readlane(incl, 63);
    if (u < base + total) {
      const unsigned long long hit = __ballot(base + incl > u);
      const int idx = __ffsll((long long)hit) - 1;
      const int32_t start = base + __builtin_amdgcn_readlane(incl - cnt, idx);
      const int32_t nsr = __builtin_amdgcn_readlane(ns, idx);
      const int32_t loc = u - start;
      out->r = r0 + idx;
      out->qt = loc / nsr;
      out->s = loc % nsr;
      out->nsplit = nsr;
      out->first = start + out->qt * nsr;
      out->clen = __builtin_amdgcn_readlane(q.clen, idx);
      out->blen = __builtin_amdgcn_readlane(q.blen, idx);
      out->lo = __builtin_amdgcn_readlane(q.lo, idx);
      out->csz = __builtin_amdgcn_readlane(req_split_size(q, ns), idx);
      out->ctx0 = __builtin_amdgcn_readlane(q.c0, idx);
      out->blk0 = __builtin_amdgcn_readlane(q.b0, idx);
      return true;
    }
    base += total;
  }
  return false;
}

// Physical 16-byte chunk of logical chunk c in LDS row `row`: XOR with a
// row-dependent mask (its own inverse). K rows are read 16 rows x one chunk at
// a time (b128), so the 16 rows of a sub-tile must hit distinct 16-byte bank
// groups. V rows are read by the transpose loads 4 rows x 32 bytes per 16
// lanes; the V mask keeps chunk pairs adjacent and gives the 8 rows read
// by 32 lanes distinct 32-byte bank windows.
template <int DH>
__device__ __forceinline__ int swz_k(int row, int c) {
  if constexpr (DH == 128) return c ^ (row & 15);
  else return c ^ ((row >> 1) & 7);
}
template <int DH>
__device__ __forceinline__ int swz_v(int row, int c) {
  if constexpr (DH == 128) return c ^ ((row & 7) << 1);
  else return c ^ (((row >> 1) & 3) << 1);
}

__device__ __forceinline__ int32_t uni(int32_t x) { return __builtin_amdgcn_readfirstlane(x); }

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their no-wait maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// Workgroup barrier without the memory fence __syncthreads() carries (that
// fence would drain every outstanding load, including prefetched tiles).
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS stages of the main kernel (NSTAGE - 1 tiles in flight). A launch of
// one round of two workgroups per CU runs 3 (four tiles in flight per CU;
// measured 96.9 vs 99.1 us on 4 x 32768 context rows and 56.4 vs 57.1 us on
// the 16-request sliding-window batch); one workgroup per CU (fewer units) or
// several rounds (many requests) run 4 (3 stages measured 20.1 vs 19.8 and
// 115.1 vs 113.6 us there), and so does any block that may span three tiles:
// the fused prologue normalises the block's K rows in the stages of its first
// tiles before the loop.
constexpr int NSTAGE_MAX = 4;
constexpr int MAX_BLK_3STAGE = KT + 1;  // block rows that span at most two tiles

// s_waitcnt takes an immediate: wait until at most k * STEP vector-memory
// operations are outstanding, for a run-time k (clamped to [0, MAXK]).
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

// Per-head RMSNorm + NeoX RoPE of one head vector held by the four lanes
// {m, m+16, m+32, m+48} in the MFMA operand layout: this lane holds chunks
// j + 4 ds (ds < DS) of 8 elements, i.e. d = 8 (j + 4 ds) + e; chunk ds pairs
// with chunk ds + DS/2 (d and d + Dh/2). Same arithmetic as qk_norm_rope_kernel:
// y = x * (1/rms) * w, then (y_lo c - y_hi s, y_hi c + y_lo s), rounded once.
// The operands (weights of the lane's dims, cos/sin of its pairs at the row's
// position) are loaded apart from the arithmetic, so that the kernel can
// issue those loads while its first tile copies are in flight.
template <int DH>
struct RopeOps {
  float wlo[DH / 64][8], whi[DH / 64][8], c[DH / 64][8], sn[DH / 64][8];
};

template <int DH>
__device__ __forceinline__ void load_rope_weights(const float* w, int j, RopeOps<DH>& o) {
#pragma unroll
  for (int ds = 0; ds < DH / 64; ++ds) {
    const int dlo = 8 * (j + 4 * ds);
    const float4* wl = reinterpret_cast<const float4*>(w + dlo);
    const float4* wh = reinterpret_cast<const float4*>(w + dlo + DH / 2);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float4 l = wl[h], u = wh[h];
      o.wlo[ds][4 * h] = l.x; o.wlo[ds][4 * h + 1] = l.y; o.wlo[ds][4 * h + 2] = l.z; o.wlo[ds][4 * h + 3] = l.w;
      o.whi[ds][4 * h] = u.x; o.whi[ds][4 * h + 1] = u.y; o.whi[ds][4 * h + 2] = u.z; o.whi[ds][4 * h + 3] = u.w;
    }
  }
}

template <int DH>
__device__ __forceinline__ void load_rope_cs(const float2* cs, int j, RopeOps<DH>& o) {
#pragma unroll
  for (int ds = 0; ds < DH / 64; ++ds) {
    const float4* c4 = reinterpret_cast<const float4*>(cs + 8 * (j + 4 * ds));
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float4 v = c4[h];
      o.c[ds][2 * h] = v.x; o.sn[ds][2 * h] = v.y; o.c[ds][2 * h + 1] = v.z; o.sn[ds][2 * h + 1] = v.w;
    }
  }
}

template <int DH>
__device__ __forceinline__ void apply_norm_rope(const bf16x8 (&xin)[DH / 32], const RopeOps<DH>& o,
                                                float eps, bf16x8 (&out)[DH / 32]) {
  constexpr int DS = DH / 32;
  float x[DS][8];
  float ss = 0.f;
#pragma unroll
  for (int ds = 0; ds < DS; ++ds)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[ds][e] = bf2f(xin[ds][e]);
      ss += x[ds][e] * x[ds][e];
    }
  ss = xrow4_sum(ss);
  const float inv = 1.0f / sqrtf(ss * (1.0f / DH) + eps);
#pragma unroll
  for (int ds = 0; ds < DS / 2; ++ds)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float lo = x[ds][e] * inv * o.wlo[ds][e];
      const float hi = x[ds + DS / 2][e] * inv * o.whi[ds][e];
      out[ds][e] = f2bf(lo * o.c[ds][e] - hi * o.sn[ds][e]);
      out[ds + DS / 2][e] = f2bf(hi * o.c[ds][e] + lo * o.sn[ds][e]);
    }
}

// Pool row of context key k of a unit over a paged store, from the page ids
// the unit staged in LDS (s_pg[i] = page of keys [PAGE (pfirst + i), ...));
// both the LDS index and the page id are clamped into range.
__device__ __forceinline__ int64_t paged_row(const int32_t* s_pg, int32_t k, int32_t pfirst,
                                             int32_t num_pages_m1) {
  const int32_t i = min(max(k / PAGE - pfirst, 0), PG_MAX - 1);
  const int32_t pid = min(max(s_pg[i], 0), num_pages_m1);
  return (int64_t)pid * PAGE + (k % PAGE);
}

__device__ __forceinline__ int32_t clamp_pos(int32_t p, int32_t max_pos) {
  return p < 0 ? 0 : (p >= max_pos ? max_pos - 1 : p);
}

// Two workgroups (8 waves) per CU at this kernel's LDS use, so up to 256
// VGPRs per wave are free; saying so keeps the compiler from spilling to
// stay under the 4-wave budget (a scratch reload inside the loop would wait
// for every tile copy in flight).
template <int DH, bool FUSE, int NSTAGE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 2))) void block_attn_bf16_kernel(AttnArgs a) {
  constexpr int CH = DH / 8;                 // 16-byte chunks per row
  constexpr int DS = DH / 32;                // MFMA k-steps over the head dim
  constexpr int DT = DH / 16;                // 16-wide d tiles of O^T
  constexpr int ROWS_PER_INST = 64 / CH;     // rows one wave-wide 16-byte load fills (1 KB)
  constexpr int LPW = KT / ROWS_PER_INST / 4;  // such loads per wave per tensor per tile
  constexpr int LPT = 2 * LPW;               // per thread per tile (K and V)
  constexpr int TILE_ELEMS = KT * DH;
  constexpr int STAGE_ELEMS = 2 * TILE_ELEMS;
  static_assert(LPW >= 1, "tile too small");
  extern __shared__ __attribute__((aligned(16))) bf16 smem[];  // [stage][K | V][KT][DH]

  // read together before any branch (one scalar round trip)
  // Launched as (kv-head, unit) = (blockIdx.x, blockIdx.y + 65535 blockIdx.z):
  // the unit index needs no argument read. With the host plan, the launch-order
  // entry (a scalar load) and, lane l, request l's record are read together
  // with the plan's counts, all before any branch, and the unit's request is
  // then read from its lane: the unit's numbers arrive after one memory round
  // trip.
  const uint64_t pt0 = pt_now();
  const int32_t g = blockIdx.x;
  int32_t u = (int32_t)blockIdx.y + 65535 * (int32_t)blockIdx.z;  // canonical unit index
  const int32_t hnreq = a.hs.nreq, hnunits = a.hs.nunits;
  const int32_t e = a.hs.order[min(u, HS_MAX_UNITS - 1)];
  const ReqSched q = a.hs.req[threadIdx.x & 63];
  const int32_t hr = e >> 8;
  // every field read from the unit's lane before any branch, so that the
  // loads above are all issued ahead of one wait
  auto pick = [&](int32_t v) { return __builtin_amdgcn_readlane(v, hr & (HS_MAX_REQS - 1)); };
  const int32_t h_ns = pick(q.ns), h_ubase = pick(q.ubase), h_clen = pick(q.clen);
  const int32_t h_blen = pick(q.blen), h_lo = pick(q.lo), h_csz = pick(q.csz);
  const int32_t h_c0 = pick(q.c0), h_b0 = pick(q.b0);
  // The arguments the prologue and the first copies need, read here with the
  // lookup (one batch of scalar loads and one wait) rather than each at its
  // first use behind a branch (a dependent argument read each).
  asm volatile("" ::"s"(a.q), "s"(a.kb), "s"(a.vb), "s"(a.kc), "s"(a.vc), "s"(a.bt), "s"(a.bpos),
               "s"(a.rope), "s"(a.qnw), "s"(a.knw), "s"(a.total_blk), "s"(a.hq), "s"(a.hkv),
               "s"(a.group), "s"(a.max_blk), "s"(a.max_pos), "s"(a.eps), "s"(a.causal),
               "s"(a.window), "s"(a.scale_log2), "s"(a.bt_stride), "s"(a.num_pages_m1));
  const bool host_plan = hnreq > 0;
  // (no short circuit, so that every load above stays ahead of the branch)
  if (host_plan & ((u >= hnunits) | (hr >= HS_MAX_REQS))) return;
  Unit un;
  if (host_plan) {
    // planned on the host: the unit's request and its numbers are kernel arguments
    const int32_t loc = e & 255;
    const int32_t ns = h_ns, ubase = h_ubase;
    u = ubase + loc;
    un.r = hr;
    un.qt = loc / ns;
    un.s = loc - un.qt * ns;
    un.nsplit = ns;
    un.first = ubase + un.qt * ns;
    un.clen = h_clen; un.blen = h_blen; un.lo = h_lo; un.csz = h_csz;
    un.ctx0 = h_c0; un.blk0 = h_b0;
  } else {
    const ReqView rv(a);
    const int32_t chunk = __builtin_amdgcn_readfirstlane(choose_chunk(a, rv));
    if (g == 0 && u == 0 && threadIdx.x == 0) a.hdr[0] = chunk;  // for the merge kernel
    if (!find_unit(a, rv, chunk, u, &un)) return;  // uniform over the workgroup
  }
  // Every lane holds the same unit; say so to the compiler (scalar registers,
  // scalar branches).
  un.r = uni(un.r); un.qt = uni(un.qt); un.s = uni(un.s); un.nsplit = uni(un.nsplit);
  un.first = uni(un.first); un.clen = uni(un.clen); un.blen = uni(un.blen); un.lo = uni(un.lo);
  un.csz = uni(un.csz);
  un.ctx0 = uni(un.ctx0); un.blk0 = uni(un.blk0);
  const uint64_t pt1 = pt_now();
  uint64_t* const pt_rec =
      kPhaseTrace ? a.trace + 8 * (((int64_t)blockIdx.y + 65535 * (int64_t)blockIdx.z) * gridDim.x + blockIdx.x)
                  : nullptr;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int m = lane & 15;   // query row within the wave / MFMA column
  const int j = lane >> 4;   // lane group

  const int32_t n_all = un.clen + un.blen;
  const int32_t k_begin = un.lo + un.s * un.csz;
  const int32_t k_end = min(k_begin + un.csz, n_all);
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

  // With the fused prologue the tiles that hold block keys are visited first
  // (the softmax is order-free), so their K rows can be normalised in LDS
  // before the loop. kb_first / nblk: the unit's block rows.
  const int32_t kb_first = max(k_begin, un.clen);
  const int32_t nblk = FUSE ? max(0, k_end - kb_first) : 0;
  const int32_t rot = nblk > 0 ? (kb_first - k_begin) / KT : 0;
  auto tile_k0 = [&](int32_t it) {
    int32_t t = it + rot;
    if (t >= ntiles) t -= ntiles;
    return k_begin + t * KT;
  };

  // Block rows of the fused prologue: this lane's query row b and the block
  // K row (16 w + m) it normalises, as indices into the unit's block rows.
  const int32_t krho = 16 * w + m;
  const int32_t kb_row = (kb_first - un.clen) + krho;

  bf16x8 qf[DS];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) {
    if (rvalid)
      qf[ds] = *reinterpret_cast<const bf16x8*>(a.q + (qrow * a.hq + qhead) * DH + (j + 4 * ds) * 8);
    else
      qf[ds] = bf16x8{};
  }

  // Tile loader: direct global -> LDS copies. One wave-wide load fills 1 KB of
  // LDS (ROWS_PER_INST rows) in lane order, so each lane fetches the logical
  // chunk that the swizzle places at its slot. A lane's row inside the tile
  // and its chunks are fixed, so only the tile's uniform base changes. Tiles
  // wholly inside the context (or wholly inside the block) take that path;
  // a tile that straddles the two or runs past the range end resolves each
  // lane's key, re-reading the last valid key for positions past the end
  // (finite data whose scores are masked to -inf).
  const int32_t rstride = a.hkv * DH;
  const bf16* kc_g = a.kc + (int64_t)g * DH;
  const bf16* vc_g = a.vc + (int64_t)g * DH;
  const bf16* kb_g = a.kb + (int64_t)g * DH;
  const bf16* vb_g = a.vb + (int64_t)g * DH;
  int lrow[LPW], koff[LPW], voff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int q = w * LPW + i;
    lrow[i] = q * ROWS_PER_INST + lane / CH;
    koff[i] = lrow[i] * rstride + swz_k<DH>(lrow[i], lane % CH) * 8;
    voff[i] = lrow[i] * rstride + swz_v<DH>(lrow[i], lane % CH) * 8;
  }
  // Paged context: the unit's page ids are staged in LDS (after the stages)
  // before the first tile copy; context row k of the unit then lives at pool
  // row s_pg[k / PAGE - pfirst] * PAGE + k % PAGE.
  const bool paged = a.bt != nullptr;
  int32_t* const s_pg = reinterpret_cast<int32_t*>(smem + NSTAGE * STAGE_ELEMS);
  // Fused prologue: each wave's own copy of the positions of the unit's block
  // rows (lane i: block row i; the prologue requires at most 64 of them).
  int32_t* const s_pos = s_pg + PG_MAX + 64 * w;
  const int32_t kc_end = min(k_end, un.clen);
  const int32_t pfirst = k_begin / PAGE;
  const int32_t npg = (paged && kc_end > k_begin) ? (kc_end - 1) / PAGE - pfirst + 1 : 0;
  const int32_t ctx0 = un.ctx0, np_m1 = a.num_pages_m1;
  // The copies are issued through inline assembly: the compiler's wait
  // insertion cannot tell which LDS stage a later LDS read touches and would
  // otherwise drain every copy in flight before it. All waits on these copies
  // are explicit (wait_vmcnt below); no other vector-memory load is in flight
  // while they are. Each K/V byte is read once per call, so the copies carry
  // the non-temporal hint (measured 3-11% faster per call than the default
  // policy).
  auto dma = [](const bf16* src, bf16* dst) {
    const uint32_t lds_addr =
        __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(DF_LDS void*)dst);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt"
                 :
                 : "s"(lds_addr), "v"(src)
                 : "memory", "m0");
  };
  auto issue_tile = [&](int32_t t) {
    const int32_t kt0 = tile_k0(t);
    bf16* st = smem + (t % NSTAGE) * STAGE_ELEMS;
    if (kt0 + KT <= min(un.clen, k_end)) {
      if (!paged) {
        const int64_t base = (int64_t)(un.ctx0 + kt0) * rstride;
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
          const int q = w * LPW + i;
          dma(kc_g + base + koff[i], st + q * 512);
          dma(vc_g + base + voff[i], st + TILE_ELEMS + q * 512);
        }
      } else {
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
          const int q = w * LPW + i;
          const int64_t rbase = (paged_row(s_pg, kt0 + lrow[i], pfirst, np_m1) - lrow[i]) * rstride;
          dma(kc_g + rbase + koff[i], st + q * 512);
          dma(vc_g + rbase + voff[i], st + TILE_ELEMS + q * 512);
        }
      }
    } else if (kt0 >= un.clen && kt0 + KT <= k_end) {
      const int64_t base = (int64_t)(un.blk0 + kt0 - un.clen) * rstride;
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int q = w * LPW + i;
        dma(kb_g + base + koff[i], st + q * 512);
        dma(vb_g + base + voff[i], st + TILE_ELEMS + q * 512);
      }
    } else {
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int q = w * LPW + i;
        const int32_t kidx = min(kt0 + lrow[i], k_end - 1);
        const bool in_ctx = kidx < un.clen;
        const int64_t r = in_ctx ? (paged ? paged_row(s_pg, kidx, pfirst, np_m1) : (int64_t)ctx0 + kidx)
                                 : (int64_t)un.blk0 + (kidx - un.clen);
        const int64_t rbase = (r - lrow[i]) * rstride;
        // select values, not the pointer variables themselves (a conditional of
        // the two lvalues would keep them in private memory)
        const uintptr_t ks = in_ctx ? (uintptr_t)kc_g : (uintptr_t)kb_g;
        const uintptr_t vs = in_ctx ? (uintptr_t)vc_g : (uintptr_t)vb_g;
        dma(reinterpret_cast<const bf16*>(ks) + rbase + koff[i], st + q * 512);
        dma(reinterpret_cast<const bf16*>(vs) + rbase + voff[i], st + TILE_ELEMS + q * 512);
      }
    }
  };

  f32x4 acc_o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc_o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mx = -INFINITY;  // reference max (log2 domain) of this lane's query row
  float lsum = 0.f;      // this lane's share of the running sum

  // Masking is needed on tiles with keys past the range end, or that reach
  // beyond the first query (causal) or before the last query's window.
  const int32_t qmin = un.clen;
  const int32_t qmax = un.clen + un.blen - 1;
  constexpr float TAU = 8.0f;  // rescale only when a row max grows by > 2^8

  if (npg > 0) {
    // 64 page ids per wave-wide copy (4 bytes a lane); indices past the
    // table row are clamped into it.
    const int32_t* bt_r = a.bt + (int64_t)un.r * a.bt_stride;
    for (int32_t c = w; c * 64 < npg; c += NT / 64) {
      const int32_t idx = min(pfirst + c * 64 + lane, a.bt_stride - 1);
      const uint32_t lds_addr =
          __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(DF_LDS void*)(s_pg + c * 64));
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
                   :
                   : "s"(lds_addr), "v"(bt_r + idx)
                   : "memory", "m0");
    }
    wait_vmcnt<0>();
    block_barrier();
  }
  // Operands of the fused prologue. Every row needs the norm weights and the
  // cos/sin of its position, and the unit's q rows (G heads) and block K rows
  // share the positions of its block rows. When they fit, the weights and the
  // cos/sin rows of the unit's block rows are copied once into the stage that
  // no tile occupies before the loop, [q weights | k weights | rows], and
  // every lane reads its operands from LDS; otherwise each lane loads its
  // own from global memory (per-lane loads of shared data would cost more
  // vector-memory return bandwidth than the unit's K/V tiles).
  float* const s_op = reinterpret_cast<float*>(smem + (NSTAGE - 1) * STAGE_ELEMS);
  float2* const s_cs = reinterpret_cast<float2*>(s_op + 256);
  constexpr int CPR = DH / 4;    // 16-byte chunks per cos/sin row
  constexpr int RPD = 64 / CPR;  // cos/sin rows per wave-wide copy (1 KB)
  // The rows sit CSTR float2 apart, 16 bytes more than a row: the lanes that
  // read the same pair of dims of 8 different rows then hit 8 different banks
  // (at a 512-byte stride they all hit the same one).
  constexpr int CSTR = DH / 2 + 2;
  const int32_t ncopy = (un.blen + RPD - 1) / RPD;
  const bool op_lds = FUSE && un.blen > 0 &&
                      1024 + ncopy * RPD * CSTR * (int)sizeof(float2) <= STAGE_ELEMS * (int)sizeof(bf16);
  if constexpr (FUSE) {
    // The positions travel like the tiles (a direct copy into LDS, waited on
    // explicitly), ahead of them, so that reading them waits for this copy
    // only and not for the tiles behind it.
    const int64_t pidx = max((int64_t)0, min((int64_t)un.blk0 + lane, a.total_blk - 1));
    const uint32_t lds_addr = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(DF_LDS void*)s_pos);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
                 :
                 : "s"(lds_addr), "v"(a.bpos + pidx)
                 : "memory", "m0");
    if (op_lds && w == 0) {
      // lane l: 16 bytes of the q weights (l < DH / 4), else of the k weights
      const int which = min(lane / CPR, 1);
      const float* src = (which == 0 ? a.qnw : a.knw) + (lane % CPR) * 4;
      const uint32_t lds_w = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(DF_LDS void*)s_op);
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                   :
                   : "s"(lds_w), "v"(src)
                   : "memory", "m0");
    }
  }
  const int32_t nfirst = min(ntiles, NSTAGE - 1);
#pragma unroll
  for (int t = 0; t < NSTAGE - 1; ++t)
    if (t < ntiles) issue_tile(t);
  if (FUSE && op_lds) {
    // positions landed (the tile copies issued after them may stay in
    // flight); then the cos/sin rows of the block rows, by position
    wait_vmcnt_steps<LPT, NSTAGE - 1>(nfirst);
    asm volatile("" ::: "memory");
    for (int32_t c = w; c < ncopy; c += NT / 64) {
      const int32_t row = min(c * RPD + lane / CPR, un.blen - 1);
      const int32_t pos = clamp_pos(s_pos[min(row, 63)], a.max_pos);
      const float2* src = a.rope + (int64_t)pos * (DH / 2) + (lane % CPR) * 2;
      // one copy per row (its CPR lanes active): a lane's 16 bytes land at
      // M0 + 16 * lane, so M0 is the row's slot minus its first lane's offset
#pragma unroll
      for (int g2 = 0; g2 < RPD; ++g2) {
        if (lane / CPR == g2) {
          const uint32_t lds_cs =
              __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(DF_LDS void*)(s_cs + (c * RPD + g2) * CSTR)) -
              (uint32_t)(g2 * CPR * 16);
          asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                       :
                       : "s"(lds_cs), "v"(src)
                       : "memory", "m0");
        }
      }
    }
  }
  // Settle q, the prologue operands and the first copies once, before the
  // loop; inside it the only vector-memory operations are the tile copies.
  wait_vmcnt<0>();

  if constexpr (FUSE) {
    if (op_lds) block_barrier();  // every wave's operand copies are in LDS
    RopeOps<DH> ops;              // q's operands, then the block K row's
    // q: RMSNorm + RoPE in registers (rows of this lane group).
    if (op_lds) {
      load_rope_weights<DH>(s_op, j, ops);
      load_rope_cs<DH>(s_cs + min(max(b, 0), un.blen - 1) * CSTR, j, ops);
    } else {
      const int32_t pos_q = rvalid ? s_pos[min(b, 63)] : 0;
      load_rope_weights<DH>(a.qnw, j, ops);
      load_rope_cs<DH>(a.rope + (int64_t)clamp_pos(pos_q, a.max_pos) * (DH / 2), j, ops);
    }
    bf16x8 qn[DS];
    apply_norm_rope<DH>(qf, ops, a.eps, qn);
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) qf[ds] = rvalid ? qn[ds] : bf16x8{};
    // block K rows: in place in the LDS stages of the first tiles (at most
    // NSTAGE - 1 of them hold block keys: the host picks NSTAGE for the
    // longest block).
    if (nblk > 0) {
      wait_lgkm0();
      block_barrier();
      const bool kv = krho < nblk;
      const int32_t kidx = kb_first + (kv ? krho : 0);
      const int32_t itk = (kidx - k_begin) / KT - rot;  // iteration that holds it
      const int row = (kidx - k_begin) % KT;
      bf16* kr = smem + itk * STAGE_ELEMS + row * DH;
      bf16x8 kx[DS], ky[DS];
#pragma unroll
      for (int ds = 0; ds < DS; ++ds)
        kx[ds] = kv ? *reinterpret_cast<const bf16x8*>(kr + swz_k<DH>(row, j + 4 * ds) * 8) : bf16x8{};
      if (op_lds) {
        load_rope_weights<DH>(s_op + DH, j, ops);
        load_rope_cs<DH>(s_cs + min(max(kb_row, 0), un.blen - 1) * CSTR, j, ops);
      } else {
        const int32_t pos_k = kv ? s_pos[min(kb_row, 63)] : 0;
        load_rope_weights<DH>(a.knw, j, ops);
        load_rope_cs<DH>(a.rope + (int64_t)clamp_pos(pos_k, a.max_pos) * (DH / 2), j, ops);
      }
      apply_norm_rope<DH>(kx, ops, a.eps, ky);
      if (kv) {
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
          *reinterpret_cast<bf16x8*>(kr + swz_k<DH>(row, j + 4 * ds) * 8) = ky[ds];
      }
    }
  }

  const int src_row = 4 * j + (m >> 2);
  const int src_col4 = (m & 3) * 4;

  const uint64_t pt2 = pt_now();
  for (int32_t it = 0; it < ntiles; ++it) {
    // Own loads of tile `it` landed (tiles issued after it may stay in flight),
    // then the barrier makes every wave's part visible and frees stage it-1.
    // With two workgroups per CU in one round (the three-stage launches) a
    // SIMD runs one wave of each; the wave that is about to issue the next
    // copies goes first (measured 95.7 -> 94.6 us on config 5, 55.8 -> 55.4 on
    // config 4; with one workgroup per CU, or several rounds, it measured
    // 0.2 us slower, so those launches leave priorities alone).
    if constexpr (NSTAGE == 3) __builtin_amdgcn_s_setprio(1);
    wait_vmcnt_steps<LPT, NSTAGE - 2>(ntiles - 1 - it);
    wait_lgkm0();
    block_barrier();
    if (it + NSTAGE - 1 < ntiles) issue_tile(it + NSTAGE - 1);
    if constexpr (NSTAGE == 3) __builtin_amdgcn_s_setprio(0);

    const int32_t kt0 = tile_k0(it);
    const bf16* kd = smem + (it % NSTAGE) * STAGE_ELEMS;
    const bf16* vd = kd + TILE_ELEMS;

    // S^T = K Q^T for the two sub-tiles of 16 keys (all K fragments first).
    bf16x8 kf[2][DS];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        const int row = 16 * t + m;
        kf[t][ds] = *reinterpret_cast<const bf16x8*>(kd + row * DH + swz_k<DH>(row, j + 4 * ds) * 8);
      }
    f32x4 sacc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < DS; ++ds)
        sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[t][ds], qf[ds], sacc[t], 0, 0, 0);
    }

    // Online softmax on this lane's 8 keys (16t + 4j + i) of query row m.
    const bool need_mask = (kt0 + KT > k_end) ||
                           (a.causal && (kt0 + KT - 1 > qmin ||
                                         (a.window > 0 && kt0 <= qmax - a.window)));
    float sv[2][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
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
    // Rescale only when some row's max outgrew the reference by > TAU; the
    // exponentials stay <= 2^TAU otherwise. Exact: the same reference max is
    // used for the sum and the accumulator.
    if (__ballot(tmax > mx + TAU)) {
      const float mnew = fmaxf(mx, tmax);
      const float alpha = (mnew == -INFINITY) ? 1.f : fast_exp2(mx - mnew);
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc_o[dt] = acc_o[dt] * alpha;
      mx = mnew;
    }
    const float msafe = (mx == -INFINITY) ? 0.f : mx;
    bf16x8 pf;
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = fast_exp2(sv[t][i] - msafe);
        psum += p;
        pf[4 * t + i] = f2bf(p);
      }
    lsum += psum;

    // O^T += V^T P^T over the 32 keys. The transpose read hands lane i of
    // group j column (16dt + i) of rows key(j, e); source lane s supplies row
    // 16h + 4j + s/4 at columns 16dt + 4(s%4) .. +3.
    bf16x8 vf[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = 16 * h + src_row;
        const int col = 16 * dt + src_col4;
        const int off = row * DH + swz_v<DH>(row, col >> 3) * 8 + (col & 7);
        const i16x4 tv = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (DF_LDS i16x4*)((DF_LDS bf16*)(vd + off)));
        const bf16x4 bv = __builtin_bit_cast(bf16x4, tv);
#pragma unroll
        for (int e = 0; e < 4; ++e) vf[dt][4 * h + e] = bv[e];
      }
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      acc_o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], pf, acc_o[dt], 0, 0, 0);
  }

  const float ltot = xrow4_sum(lsum);
  const int32_t nrow_unit = 16 * w + m;  // row within the unit's query tile
  const uint64_t pt3 = pt_now();

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
    pt_record(pt_rec, pt0, pt1, pt2, pt3, ntiles, 1);
    return;
  }

  // Split: publish the partial: the split's own softmax output O / l (a
  // convex combination of V rows) times 2^-e in fp16, with its reference max,
  // sum and e in f32. e is chosen per query row so that the row's largest
  // magnitude lands in [2^13, 2^14): fp16 then holds any finite bf16 V range
  // without overflow and keeps 11 significant bits relative to the row's
  // largest value (8x finer than the bf16 output), however large or small V
  // is. The merge kernel that follows on the stream combines the splits.
  {
    const int64_t slot = (int64_t)u * a.hkv + g;
    f16* po = a.part_o + (slot * QROWS + nrow_unit) * DH + 4 * j;
    const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
    float amax = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(acc_o[dt][i]));
    amax = xrow4_max(amax) * inv;
    int ex = 0;
    if (amax > 0.f && amax <= 3.0e38f) {
      (void)frexpf(amax, &ex);  // amax < 2^ex
      ex -= 14;
    }
    const float sc = ldexpf(inv, -ex);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      f16x4 h;
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = (f16)(acc_o[dt][i] * sc);
      *reinterpret_cast<f16x4*>(po + 16 * dt) = h;
    }
    if (j == 0) {
      float4* pml = reinterpret_cast<float4*>(a.part_ml) + slot * QROWS + nrow_unit;
      *pml = make_float4(mx, ltot, (float)ex, 0.f);
    }
    if (un.s == 0 && tid == 0 && a.hs.nreq == 0)
      a.dir[((int64_t)un.r * a.qtiles + un.qt) * a.hkv + g] = un.first;
  }
  pt_record(pt_rec, pt0, pt1, pt2, pt3, ntiles, 1);
}

// Streaming log-sum-exp over a row's ns split partials in index order, MB
// splits per batch (their loads issued together): the row's running max M,
// sum L and output o. Split s's record sits at ml_row[s * sstride] and its
// values at ov_row[s * sstride * DH].
template <int MB, int DV, int DH>
__device__ __forceinline__ void merge_splits(const float4* ml_row, const f16* ov_row, int64_t sstride,
                                             int32_t ns, float& M, float& L, float (&o)[DV]) {
  for (int32_t s0 = 0; s0 < ns; s0 += MB) {
    float4 ml[MB];
    f16x8 ov[MB];
#pragma unroll
    for (int bb = 0; bb < MB; ++bb) {
      const int64_t sidx = s0 + bb < ns ? s0 + bb : ns - 1;
      ml[bb] = ml_row[sidx * sstride];
      ov[bb] = *reinterpret_cast<const f16x8*>(ov_row + sidx * sstride * DH);
    }
    float bm = M;
#pragma unroll
    for (int bb = 0; bb < MB; ++bb)
      if (s0 + bb < ns) bm = fmaxf(bm, ml[bb].x);
    const float bsafe = (bm == -INFINITY) ? 0.f : bm;
    const float rescale = fast_exp2(M - bsafe);
    L *= rescale;
#pragma unroll
    for (int d = 0; d < DV; ++d) o[d] *= rescale;
#pragma unroll
    for (int bb = 0; bb < MB; ++bb) {
      // split weight: its sum l times 2^(m - M); its values are O / l stored
      // times 2^-e
      const float wgt = (s0 + bb < ns) ? ml[bb].y * fast_exp2(ml[bb].x - bsafe) : 0.f;
      const float wov = ldexpf(wgt, (int)ml[bb].z);
      L += wgt;
#pragma unroll
      for (int d = 0; d < DV; ++d) o[d] += (float)ov[bb][d] * wov;
    }
    M = bm;
  }
}

// Merge of split partials: one workgroup per (request, query tile, kv-head,
// block of MROWS rows); thread -> (row, 8 head-dim values). Splits are
// consumed in index order by a streaming log-sum-exp, MB at a time with their
// loads in flight, so the result does not depend on scheduling.
constexpr int MROWS = 16;
template <int DH>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 2))) void block_attn_merge_kernel(AttnArgs a) {
  constexpr int DV = 8;                   // head-dim values per thread
  constexpr int TPR = DH / DV;            // threads per row
  constexpr int RPW = NT / TPR;           // rows per workgroup pass
  const int32_t rb_count = QROWS / MROWS;
  const uint64_t pt0 = pt_now();
  // What the host-planned path needs is read before any branch: the scalar
  // arguments and, lane l, request l's record (zeros past the requests), so
  // one memory round trip precedes the partials' loads.
  const int32_t hkv = a.hkv, qtiles = a.qtiles, nreqs = a.num_reqs, hplan = a.hplan;
  const int32_t group = a.group;
  const ReqSched ql = a.hs.req[threadIdx.x & 63];
  int64_t id = blockIdx.x;
  const int32_t rb = (int32_t)(id % rb_count); id /= rb_count;
  const int32_t g = (int32_t)(id % hkv); id /= hkv;
  const int32_t qt = (int32_t)(id % qtiles); id /= qtiles;
  const int32_t r = (int32_t)id;
  const int32_t rl = min(r, HS_MAX_REQS - 1);
  const int32_t h_ns = __builtin_amdgcn_readlane(ql.ns, rl);
  const int32_t h_blen = __builtin_amdgcn_readlane(ql.blen, rl);
  const int32_t h_b0 = __builtin_amdgcn_readlane(ql.b0, rl);
  const int32_t h_ubase = __builtin_amdgcn_readlane(ql.ubase, rl);
  // (the pointers and sizes of the merge itself, read in the same batch)
  asm volatile("" ::"s"(a.part_o), "s"(a.part_ml), "s"(a.out), "s"(a.total_blk), "s"(a.hq),
               "s"(a.num_reqs), "s"(a.hplan), "s"(a.qtiles), "s"(a.hkv), "s"(a.group));
  // host plan: unsplit sets wrote their output directly
  const bool done = (r >= nreqs) | ((hplan > 0) & ((h_ns <= 1) | (qt * QROWS >= group * h_blen)));
  if (done) return;
  int32_t ns, blen, b0, first;
  if (hplan > 0) {
    ns = h_ns; blen = h_blen; b0 = h_b0;
    first = h_ubase + qt * ns;
  } else {
    // The split size (chosen by the main kernel of this call unless fixed), the
    // directory entry and the lengths are independent loads.
    const int32_t chunk = a.chunk > 0 ? a.chunk : a.hdr[0];
    first = a.dir[((int64_t)r * qtiles + qt) * hkv + g];
    const LaneReq q = lane_req(a, r);
    if (chunk < KT) return;
    ns = req_splits(q, chunk); blen = q.blen; b0 = q.b0;
    if (ns <= 1 || qt >= q.nq) return;  // unsplit units wrote their output directly
    if (first < 0 || first + ns > a.units) return;
  }
  const int32_t nrows = a.group * blen;
  const int tid = threadIdx.x;
  const float4* pml = reinterpret_cast<const float4*>(a.part_ml);
  constexpr int PASSES = (MROWS + RPW - 1) / RPW;
#pragma unroll
  for (int pass = 0; pass < PASSES; ++pass) {
    const int rloc = pass * RPW + tid / TPR;
    if (rloc >= MROWS) break;
    const int row = rb * MROWS + rloc;
    const int d0 = (tid % TPR) * DV;
    const int32_t nq2 = qt * QROWS + row;
    float o[DV];
#pragma unroll
    for (int d = 0; d < DV; ++d) o[d] = 0.f;
    float M = -INFINITY, L = 0.f;
    // The splits in batches of MB whose loads are in flight together: MB = 8
    // up to 8 splits, else 16 (one memory round trip for up to 16 splits at
    // the cost of more registers). The batch size depends on the split count
    // only, so every plan that splits a request the same way gives the same
    // bits.
    const float4* ml_row = pml + (int64_t)first * a.hkv * QROWS + (int64_t)g * QROWS + row;
    const f16* ov_row = a.part_o + ((int64_t)first * a.hkv * QROWS + (int64_t)g * QROWS + row) * DH + d0;
    const int64_t sstride = (int64_t)a.hkv * QROWS;  // between consecutive splits, in rows
    if (ns <= 8) merge_splits<8, DV, DH>(ml_row, ov_row, sstride, ns, M, L, o);
    else merge_splits<16, DV, DH>(ml_row, ov_row, sstride, ns, M, L, o);
    if (nq2 < nrows) {
      const int32_t hl2 = nq2 / blen;
      const int32_t b2 = nq2 - hl2 * blen;
      const int64_t qrow2 = (int64_t)b0 + b2;
      if (qrow2 < a.total_blk) {
        const float inv = L > 0.f ? 1.0f / L : 0.f;
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < DV; ++e) v[e] = f2bf(o[e] * inv);
        *reinterpret_cast<bf16x8*>(a.out + (qrow2 * a.hq + g * a.group + hl2) * DH + d0) = v;
      }
    }
  }
  pt_record(a.trace + 8 * (a.trace_main + blockIdx.x), pt0, 0, 0, 0, ns, 2);
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
  const int32_t* bt;  // paged context store (nullptr: packed rows)
  int32_t bt_stride, num_pages_m1;
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
        int64_t row = (int64_t)c0 + kidx;
        bool ok = row < a.total_ctx;
        if (a.bt) {
          const int32_t pid = min(max(a.bt[(int64_t)r * a.bt_stride + min(kidx / PAGE, a.bt_stride - 1)], 0),
                                  a.num_pages_m1);
          row = (int64_t)pid * PAGE + kidx % PAGE;
          ok = true;
        }
        if (ok) { krow = a.kc + (row * a.hkv + g) * DH; vrow_mine = a.vc + (row * a.hkv + g) * DH; }
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

// Host mirror of lane_req / choose_chunk / find_unit's numbering: the same
// integer arithmetic on the host copies of the lengths, so the plan (and the
// result) is the one the kernels would derive on the device.
struct HostReq {
  int32_t c0, b0, clen, blen, lo, n, nq;
};
HostReq host_req(const dflash_block_attn_params& p, int32_t group, int32_t r) {
  const int32_t* hc = p.host_cu_ctx_lens;
  const int32_t* hb = p.host_cu_blk_lens;
  const int32_t tc = (int32_t)p.total_ctx, tb = (int32_t)p.total_blk;
  HostReq q{};
  q.c0 = std::min(std::max(hc[r], 0), tc);
  const int32_t c1 = std::min(std::max(hc[r + 1], q.c0), tc);
  q.b0 = std::min(std::max(hb[r], 0), tb);
  const int32_t b1 = std::min(std::max(hb[r + 1], q.b0), tb);
  q.clen = c1 - q.c0;
  q.blen = std::min(b1 - q.b0, p.max_blk_len);
  q.lo = (p.causal && p.window > 0) ? std::max(q.clen - p.window + 1, 0) : 0;
  q.n = q.blen > 0 ? q.clen + q.blen - q.lo : 0;
  q.nq = q.blen > 0 ? (group * q.blen + QROWS - 1) / QROWS : 0;
  return q;
}
int32_t host_splits(const HostReq& q, int32_t chunk) {
  return q.n > 0 ? (q.n + chunk - 1) / chunk : 0;
}
int32_t host_split_size(const HostReq& q, int32_t ns) {
  return ns > 0 ? ((q.n + ns - 1) / ns + KT - 1) / KT * KT : 0;
}
int32_t host_choose_chunk(const HostReq* rq, int32_t nreq, int32_t units) {
  auto count = [&](int32_t c) {
    int64_t tot = 0;
    for (int32_t r = 0; r < nreq; ++r) tot += (int64_t)host_splits(rq[r], c) * rq[r].nq;
    return tot;
  };
  int32_t maxn = 0;
  int64_t work = 0;
  for (int32_t r = 0; r < nreq; ++r) {
    maxn = std::max(maxn, rq[r].n);
    work += (int64_t)((rq[r].n + KT - 1) / KT) * rq[r].nq;
  }
  const int32_t kmax = std::max(1, (maxn + KT - 1) / KT);
  int32_t klo = (int32_t)std::max<int64_t>(
      1, std::min<int64_t>(kmax, (work + units - 1) / std::max(units, 1)));
  if (count(klo * KT) <= units) return klo * KT;
  int32_t khi = klo, step = 1;
  while (khi < kmax) {
    khi = std::min(kmax, khi + step);
    step *= 2;
    if (count(khi * KT) <= units) break;
    klo = khi;
  }
  while (khi - klo > 1) {
    const int32_t mid = (klo + khi) / 2;
    if (count(mid * KT) <= units) khi = mid; else klo = mid;
  }
  return khi * KT;
}
// Fill hs from the host lengths; false (hs->nreq = 0) when they are absent or
// the plan does not fit the table.
bool plan_host_schedule(const dflash_block_attn_params& p, const AttnPlan& plan, bool paged,
                        HostSched* hs) {
  hs->nreq = 0;
  if (!p.host_cu_ctx_lens || !p.host_cu_blk_lens) return false;
  if (p.num_reqs > HS_MAX_REQS || plan.units > INT32_MAX) return false;
  HostReq rq[HS_MAX_REQS];
  for (int32_t r = 0; r < p.num_reqs; ++r) rq[r] = host_req(p, plan.group, r);
  const int32_t units = (int32_t)plan.units;
  // same budgets, in the same order, as choose_chunk on the device
  int32_t chunk = plan.chunk;
  if (chunk <= 0) {
    const int32_t pref = (int32_t)plan.units_pref;
    chunk = host_choose_chunk(rq, p.num_reqs, pref);
    if (paged && chunk > PAGED_MAX_UNIT_KEYS && pref < units)
      chunk = host_choose_chunk(rq, p.num_reqs, units);
  }
  int32_t ubase = 0;
  // (keys, canonical index, entry) of every unit; sorted by decreasing keys
  std::pair<int32_t, int32_t> key[HS_MAX_UNITS];
  uint16_t ent[HS_MAX_UNITS];
  for (int32_t r = 0; r < p.num_reqs; ++r) {
    const int32_t ns = host_splits(rq[r], chunk);
    const int32_t cnt = ns * rq[r].nq;
    if (cnt > 256 || ubase + cnt > HS_MAX_UNITS || ubase + cnt > units) return false;
    const int32_t csz = host_split_size(rq[r], ns);
    hs->req[r] = ReqSched{rq[r].c0, rq[r].b0, rq[r].clen, rq[r].blen, rq[r].lo, csz, ns, ubase};
    for (int32_t k = 0; k < cnt; ++k) {
      const int32_t s = k % ns;
      const int32_t keys = std::min(csz, rq[r].n - s * csz);
      key[ubase + k] = {-keys, ubase + k};
      ent[ubase + k] = (uint16_t)((r << 8) | k);
    }
    ubase += cnt;
  }
  std::sort(key, key + ubase);
  for (int32_t i = 0; i < ubase; ++i) hs->order[i] = ent[key[i].second];
  hs->chunk = chunk;
  hs->nunits = ubase;
  hs->nreq = p.num_reqs;
  return true;
}

}  // namespace

bool plan_block_attention(const dflash_block_attn_params& p, int num_cus, bool paged,
                          AttnPlan* plan) {
  AttnPlan pl{};
  pl.group = p.num_q_heads / p.num_kv_heads;
  pl.cus = num_cus > 0 ? num_cus : 256;
  const int64_t qt = ((int64_t)pl.group * p.max_blk_len + QROWS - 1) / QROWS;
  pl.qtiles = (int32_t)(qt < 1 ? 1 : qt);
  int64_t eff = p.total_ctx + p.total_blk;
  if (p.causal && p.window > 0) {
    const int64_t bound = (int64_t)p.num_reqs * (p.window - 1) + p.total_blk;
    if (bound < eff) eff = bound;
  }
  if (p.split_keys > 0) {
    pl.chunk = p.split_keys;
    pl.units = (int64_t)pl.qtiles * ((eff + pl.chunk - 1) / pl.chunk + p.num_reqs);
  } else {
    // The device picks the split size (choose_chunk) so that the units fill
    // the launched grid. Resident workgroup slots: two per compute unit at
    // this kernel's LDS use. With few (request, query tile) pairs, one unit
    // per compute unit: fewer, longer splits write fewer partials for the
    // merge and spread each unit's start-up over more tiles, which measured
    // faster than filling both slots. With more pairs, one round of slots,
    // then two units per pair or two rounds.
    // Long units (over ~1536 keys at one per compute unit) fill both slots
    // instead: measured 63.0 vs 64.2 us (16 requests x 4111 keys) and 110.3
    // vs 113.0 us (4 x 32768 keys), while short ones (8 requests x ~1400
    // keys) are fastest at one unit per compute unit.
    pl.chunk = 0;
    const int64_t cus = num_cus > 0 ? num_cus : 256;
    const int64_t per_cu = std::max<int64_t>(1, cus / p.num_kv_heads);
    const int64_t slots_per_head = std::max<int64_t>(1, 2 * cus / p.num_kv_heads);
    const int64_t base = (int64_t)p.num_reqs * pl.qtiles;
    const bool long_units = eff * pl.qtiles > (int64_t)1536 * per_cu;
    pl.units = (2 * base <= per_cu && !long_units) ? per_cu
               : (2 * base <= slots_per_head)      ? slots_per_head
                                                   : std::max(2 * base, 2 * slots_per_head);
  }
  pl.units_pref = pl.units;
  if (paged && p.split_keys == 0) {
    // room for units of at most PAGED_MAX_UNIT_KEYS keys (used only when the
    // packed budget's split would be longer)
    const int64_t need = (int64_t)pl.qtiles * ((eff + PAGED_MAX_UNIT_KEYS - 1) / PAGED_MAX_UNIT_KEYS + p.num_reqs);
    pl.units = std::max(pl.units, need);
  }
  size_t off = 256;  // reserved header
  pl.off_counters = off;
  off = align_up(off + sizeof(int32_t) * (size_t)p.num_reqs * pl.qtiles * p.num_kv_heads, 256);
  pl.off_part_o = off;
  off = align_up(off + sizeof(uint16_t) * (size_t)pl.units * p.num_kv_heads * QROWS * p.head_dim, 256);
  pl.off_part_ml = off;
  off = align_up(off + sizeof(float) * 4 * (size_t)pl.units * p.num_kv_heads * QROWS, 256);
  pl.off_trace = off;
  pl.trace_main = 0;
  if (kPhaseTrace) {
    const int64_t mblocks = (int64_t)p.num_reqs * pl.qtiles * p.num_kv_heads * (QROWS / MROWS);
    pl.trace_main = pl.units * p.num_kv_heads;
    off += (size_t)64 * (size_t)(pl.trace_main + mblocks);
  }
  pl.bytes = (p.dtype == DFLASH_BF16) ? off : 0;
  *plan = pl;
  return true;
}

namespace {

// DFLASH_TRACE (environment variable, read at every call; anything but "" or
// "0"): one host-side log of each attention call's work decomposition on
// stderr: the split, the units per kv-head, the launch shapes, and per request
// (host plan) its keys, splits and split size.
bool trace_enabled() {
  const char* v = std::getenv("DFLASH_TRACE");
  return v && v[0] != '\0' && std::strcmp(v, "0") != 0;
}

void trace_plan(const dflash_block_attn_params& p, const AttnPlan& plan, const HostSched& hs,
                bool paged, bool fused, int nstage, size_t lds, dim3 grid, dim3 mgrid) {
  std::fprintf(stderr,
               "dflash trace: block_attention %s%s: %d requests, Hq %d, Hkv %d, Dh %d, %lld context "
               "rows, %lld block rows (max %d), causal %d, window %d\n",
               paged ? "paged" : "packed", fused ? " + fused q/k norm and RoPE" : "", p.num_reqs,
               p.num_q_heads, p.num_kv_heads, p.head_dim, (long long)p.total_ctx,
               (long long)p.total_blk, p.max_blk_len, p.causal, p.window);
  if (hs.nreq > 0)
    std::fprintf(stderr, "  plan: host, split %d keys, %d units per kv-head (budget %lld), %d query tiles\n",
                 hs.chunk, hs.nunits, (long long)plan.units, plan.qtiles);
  else
    std::fprintf(stderr,
                 "  plan: on the device from the device lengths (split %s), budget %lld units per "
                 "kv-head, %d query tiles\n",
                 plan.chunk > 0 ? "fixed by split_keys" : "chosen by the kernels", (long long)plan.units,
                 plan.qtiles);
  std::fprintf(stderr,
               "  launch: main grid (%u, %u, %u) x %d threads, %d LDS stages (%zu bytes); merge grid "
               "%u x %d; workspace %zu bytes\n",
               grid.x, grid.y, grid.z, NT, nstage, lds, mgrid.x, NT, plan.bytes);
  for (int32_t r = 0; r < hs.nreq; ++r) {
    const ReqSched& q = hs.req[r];
    const int32_t qt = q.blen > 0 ? (plan.group * q.blen + QROWS - 1) / QROWS : 0;
    std::fprintf(stderr,
                 "  request %d: %d context + %d block rows, keys from %d, %d split(s) of up to %d "
                 "keys x %d query tile(s)\n",
                 r, q.clen, q.blen, q.lo, q.ns, q.csz, qt);
  }
}

}  // namespace

hipError_t launch_block_attention(const dflash_block_attn_params& p, const AttnPlan& plan,
                                  const dflash_qk_prologue* pro, const dflash_paged_ctx* pg,
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
    if (pg) {
      a.bt = pg->block_table;
      a.bt_stride = pg->max_pages_per_req;
      a.num_pages_m1 = (int32_t)std::min<int64_t>(pg->num_pages - 1, INT32_MAX);
    }
    const int64_t blocks = p.total_blk * p.num_q_heads;
    if (!grid_fits(blocks)) return hipErrorInvalidConfiguration;
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
  a.dir = (int32_t*)(w + plan.off_counters);
  a.part_o = (f16*)(w + plan.off_part_o);
  a.part_ml = (float*)(w + plan.off_part_ml);
  a.total_ctx = p.total_ctx; a.total_blk = p.total_blk;
  a.num_reqs = p.num_reqs; a.hq = p.num_q_heads; a.hkv = p.num_kv_heads;
  a.group = plan.group; a.chunk = plan.chunk; a.qtiles = plan.qtiles;
  a.units = (int32_t)plan.units;
  a.units_pref = (int32_t)plan.units_pref;
  a.hdr = (int32_t*)w;
  a.trace = (uint64_t*)(w + plan.off_trace);
  a.trace_main = plan.trace_main;
  if (pg) {
    a.bt = pg->block_table;
    a.bt_stride = pg->max_pages_per_req;
    a.num_pages_m1 = (int32_t)std::min<int64_t>(pg->num_pages - 1, INT32_MAX);
  }
  if (pro) {
    a.qnw = pro->q_norm_w;
    a.knw = pro->k_norm_w;
    a.bpos = pro->positions;
    a.rope = reinterpret_cast<const float2*>(pro->rope_table);
    a.max_pos = pro->max_pos;
    a.eps = pro->eps;
  }
  a.max_blk = p.max_blk_len;
  a.scale_log2 = p.scale * LOG2E;
  a.causal = p.causal ? 1 : 0; a.window = p.window;
  plan_host_schedule(p, plan, pg != nullptr, &a.hs);
  a.hplan = a.hs.nreq;
  // Host-planned: launch only the units the plan uses.
  const int64_t blocks = (a.hs.nreq > 0 ? a.hs.nunits : plan.units) * p.num_kv_heads;
  if (blocks == 0) return hipSuccess;
  const int64_t cus = plan.cus;
  const int nstage =
      (p.max_blk_len <= MAX_BLK_3STAGE && blocks > cus && blocks <= 2 * cus) ? 3 : 4;
  const size_t lds = (size_t)nstage * 2 * KT * p.head_dim * sizeof(bf16) +
                     (PG_MAX + POS_LDS) * sizeof(int32_t);
  // The LDS limit attribute is a per-function setting: raise it once per
  // device (not per launch, so that stream capture sees only the launch).
  static std::once_flag once[64];
  int dev = 0;
  (void)hipGetDevice(&dev);
  std::call_once(once[dev & 63], [] {
    constexpr int extra = (PG_MAX + POS_LDS) * 4;
    constexpr int s128 = NSTAGE_MAX * 2 * KT * 128 * 2 + extra, s64 = NSTAGE_MAX * 2 * KT * 64 * 2 + extra;
    const void* fns[8] = {(const void*)block_attn_bf16_kernel<128, false, 3>,
                          (const void*)block_attn_bf16_kernel<128, true, 3>,
                          (const void*)block_attn_bf16_kernel<128, false, 4>,
                          (const void*)block_attn_bf16_kernel<128, true, 4>,
                          (const void*)block_attn_bf16_kernel<64, false, 3>,
                          (const void*)block_attn_bf16_kernel<64, true, 3>,
                          (const void*)block_attn_bf16_kernel<64, false, 4>,
                          (const void*)block_attn_bf16_kernel<64, true, 4>};
    for (int i = 0; i < 8; ++i)
      (void)hipFuncSetAttribute(fns[i], hipFuncAttributeMaxDynamicSharedMemorySize, i < 4 ? s128 : s64);
  });
  const int64_t mblocks = (int64_t)p.num_reqs * plan.qtiles * p.num_kv_heads * (QROWS / MROWS);
  const int64_t launch_units = blocks / p.num_kv_heads;
  // the main grid's unit index (y + 65535 z) is 32-bit, z at most 65535
  if (!grid_fits(mblocks) || !grid_fits(launch_units) || (launch_units + 65534) / 65535 > 65535)
    return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)p.num_kv_heads, (unsigned)std::min<int64_t>(launch_units, 65535),
                  (unsigned)((launch_units + 65534) / 65535));
  const dim3 blk(NT), mgrid((unsigned)mblocks);
  if (trace_enabled()) trace_plan(p, plan, a.hs, pg != nullptr, pro != nullptr, nstage, lds, grid, mgrid);
  auto launch_main = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, blk, lds, s, a); };
  if (p.head_dim == 128) {
    if (nstage == 3) {
      if (pro) launch_main(block_attn_bf16_kernel<128, true, 3>);
      else launch_main(block_attn_bf16_kernel<128, false, 3>);
    } else {
      if (pro) launch_main(block_attn_bf16_kernel<128, true, 4>);
      else launch_main(block_attn_bf16_kernel<128, false, 4>);
    }
    hipLaunchKernelGGL(block_attn_merge_kernel<128>, mgrid, blk, 0, s, a);
  } else {
    if (nstage == 3) {
      if (pro) launch_main(block_attn_bf16_kernel<64, true, 3>);
      else launch_main(block_attn_bf16_kernel<64, false, 3>);
    } else {
      if (pro) launch_main(block_attn_bf16_kernel<64, true, 4>);
      else launch_main(block_attn_bf16_kernel<64, false, 4>);
    }
    hipLaunchKernelGGL(block_attn_merge_kernel<64>, mgrid, blk, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace dflash

#ifdef DFLASH_PHASE_TRACE
// Diagnostic build only: byte offset of the phase-trace records in the
// workspace of a bf16 call with these parameters, and the number of records of
// the main kernel (the merge kernel's follow them).
extern "C" size_t dflash_phase_trace_layout(const dflash_block_attn_params* p, int paged,
                                            int64_t* main_records, int64_t* merge_records) {
  dflash::AttnPlan plan;
  dflash::plan_block_attention(*p, 256, paged != 0, &plan);
  *main_records = plan.trace_main;
  *merge_records = (int64_t)((plan.bytes - plan.off_trace) / 64) - plan.trace_main;
  return plan.off_trace;
}
#endif
