// NeoX RoPE cos/sin cache and the fused per-head q/k RMSNorm + RoPE prologue.
//
// "qwen3_dflash.cpp" page, ForwardBlockLogits: the block's q and k go through
// q_norm / k_norm (standard RMSNorm over head_dim) and then RopeNeox at the
// block positions; PrecomputeContextKVDevice applies the same k-norm + RoPE to
// the context keys. The reference runs three launches (norm q, norm k, RoPE);
// here one pass reads each head vector once, normalises it in f32, rotates it
// and writes it back.
#include "dflash_device.h"
#include "dflash_internal.h"

namespace dflash {
namespace {

// table[p][i] = (cos(p f_i), sin(p f_i)), f_i = theta^(-2i/Dh), all in f64.
__global__ void rope_table_kernel(float2* __restrict__ table, int32_t max_pos, int32_t half,
                                  double theta) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)max_pos * half) return;
  const int32_t p = (int32_t)(idx / half);
  const int32_t i = (int32_t)(idx % half);
  const double inv_freq = pow(theta, -(2.0 * (double)i) / (double)(2 * half));
  const double ang = (double)p * inv_freq;
  double s, c;
  sincos(ang, &s, &c);
  table[idx] = make_float2((float)c, (float)s);
}

// 16 bytes of T: the unit each lane loads and stores.
template <typename T>
struct Piece;
template <>
struct Piece<bf16> {
  static constexpr int N = 8;
  typedef bf16x8 raw;
  static __device__ __forceinline__ raw load(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
  static __device__ __forceinline__ float get(const raw& v, int e) { return bf2f(v[e]); }
  static __device__ __forceinline__ void store(bf16* p, const float* x) {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = f2bf(x[e]);
    *reinterpret_cast<bf16x8*>(p) = v;
  }
};
template <>
struct Piece<float> {
  static constexpr int N = 4;
  typedef f32x4 raw;
  static __device__ __forceinline__ raw load(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
  static __device__ __forceinline__ float get(const raw& v, int e) { return v[e]; }
  static __device__ __forceinline__ void store(float* p, const float* x) {
    *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
  }
};

constexpr int HC = 8;  // heads of one row per lane group

// One lane group of LANES = (DH/2) / (elements per 16 bytes) lanes takes one
// row and up to HC of its heads (q heads first, then k heads). Lane s holds
// elements [N s, N s + N) of each head's first half and their rotation
// partners DH/2 further on, so it needs the cos/sin of N frequencies only:
// those are read once per row and chunk of heads rather than once per head
// vector (per head they would be twice the bytes of the vector itself), and
// each lane has all of its heads' loads in flight together.
template <typename T, int DH>
__global__ __launch_bounds__(256) void qk_norm_rope_kernel(
    T* __restrict__ q, T* __restrict__ k, const float* __restrict__ wq,
    const float* __restrict__ wk, const int32_t* __restrict__ pos,
    const float2* __restrict__ table, int32_t max_pos, int64_t rows, int32_t hq, int32_t hkv,
    float eps) {
  // every argument in one batch of scalar loads (no dependent argument reads)
  asm volatile("" ::"s"(q), "s"(k), "s"(wq), "s"(wk), "s"(pos), "s"(table), "s"(max_pos), "s"(rows),
               "s"(hq), "s"(hkv), "s"(eps));
  constexpr int N = Piece<T>::N;
  constexpr int HALF = DH / 2;
  constexpr int LANES = HALF / N;
  constexpr int GPW = 64 / LANES;  // lane groups per wave
  const int lane = threadIdx.x & 63;
  const int s = lane % LANES;
  const int64_t grp =
      ((int64_t)blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64) * GPW + lane / LANES;
  const int32_t hq_eff = q ? hq : 0;
  const int32_t heads = hq_eff + hkv;
  const int32_t chunks = (heads + HC - 1) / HC;
  // whole lane groups leave together, so the group reductions below only
  // ever read lanes that are still running
  if (grp >= rows * chunks) return;
  const int64_t row = grp / chunks;
  const int32_t h0 = (int32_t)(grp - row * chunks) * HC;
  const int32_t p = pos[row];

  typename Piece<T>::raw x0[HC], x1[HC];
#pragma unroll
  for (int i = 0; i < HC; ++i) {
    // heads past the row's last re-read its last head and store nothing
    const int32_t h = min(h0 + i, heads - 1);
    const T* src = (h < hq_eff) ? q + (row * hq + h) * DH : k + (row * hkv + (h - hq_eff)) * DH;
    x0[i] = Piece<T>::load(src + N * s);
    x1[i] = Piece<T>::load(src + HALF + N * s);
  }
  float wa[2][N], wb[2][N];  // [q | k] weights of this lane's elements
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float* w = t == 0 ? wq : wk;
    const bool need = t == 0 ? h0 < hq_eff : h0 + HC > hq_eff;
#pragma unroll
    for (int e4 = 0; e4 < N / 4; ++e4) {
      const float4 v0 = need ? *reinterpret_cast<const float4*>(w + N * s + 4 * e4) : float4{};
      const float4 v1 = need ? *reinterpret_cast<const float4*>(w + HALF + N * s + 4 * e4) : float4{};
      wa[t][4 * e4] = v0.x; wa[t][4 * e4 + 1] = v0.y; wa[t][4 * e4 + 2] = v0.z; wa[t][4 * e4 + 3] = v0.w;
      wb[t][4 * e4] = v1.x; wb[t][4 * e4 + 1] = v1.y; wb[t][4 * e4 + 2] = v1.z; wb[t][4 * e4 + 3] = v1.w;
    }
  }
  const int32_t pc = p < 0 ? 0 : (p >= max_pos ? max_pos - 1 : p);
  const float4* cs4 = reinterpret_cast<const float4*>(table + (int64_t)pc * HALF + N * s);
  float cs[2 * N];
#pragma unroll
  for (int e2 = 0; e2 < N / 2; ++e2) {
    const float4 c = cs4[e2];
    cs[4 * e2] = c.x; cs[4 * e2 + 1] = c.y; cs[4 * e2 + 2] = c.z; cs[4 * e2 + 3] = c.w;
  }

#pragma unroll
  for (int i = 0; i < HC; ++i) {
    const int32_t h = h0 + i;
    float a[N], b[N];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < N; ++e) {
      a[e] = Piece<T>::get(x0[i], e);
      b[e] = Piece<T>::get(x1[i], e);
      ss += a[e] * a[e] + b[e] * b[e];
    }
    ss = group_sum<LANES>(ss);
    const float inv = 1.0f / sqrtf(ss * (1.0f / DH) + eps);
    const int t = h < hq_eff ? 0 : 1;
    float y0[N], y1[N];
#pragma unroll
    for (int e = 0; e < N; ++e) {
      const float u = a[e] * inv * wa[t][e];
      const float v = b[e] * inv * wb[t][e];
      const float c = cs[2 * e], sn = cs[2 * e + 1];
      y0[e] = u * c - v * sn;
      y1[e] = v * c + u * sn;
    }
    if (h < heads) {
      T* dst = (h < hq_eff) ? q + (row * hq + h) * DH : k + (row * hkv + (h - hq_eff)) * DH;
      Piece<T>::store(dst + N * s, y0);
      Piece<T>::store(dst + HALF + N * s, y1);
    }
  }
}

template <typename T, int DH>
hipError_t launch_qknr(T* q, T* k, const float* wq, const float* wk, const int32_t* pos,
                       int64_t rows, int32_t hq, int32_t hkv, float eps, const float* table,
                       int32_t max_pos, hipStream_t s) {
  const int64_t heads = (q ? hq : 0) + hkv;
  const int64_t groups = rows * ((heads + HC - 1) / HC);
  const int64_t per_block = 4 * (64 / (DH / 2 / Piece<T>::N));
  const int64_t blocks = (groups + per_block - 1) / per_block;
  if (blocks == 0) return hipGetLastError();
  if (!grid_fits(blocks)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((qk_norm_rope_kernel<T, DH>), dim3((unsigned)blocks), dim3(256), 0, s, q, k,
                     wq, wk, pos, reinterpret_cast<const float2*>(table), max_pos, rows, hq, hkv,
                     eps);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope_table(float* table, int32_t max_pos, int32_t head_dim, double theta,
                             hipStream_t s) {
  const int32_t half = head_dim / 2;
  const int64_t n = (int64_t)max_pos * half;
  const int64_t blocks = (n + 255) / 256;
  if (!grid_fits(blocks)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<float2*>(table), max_pos, half, theta);
  return hipGetLastError();
}

hipError_t launch_qk_norm_rope(dflash_dtype dt, void* q, void* k, const float* wq,
                               const float* wk, const int32_t* pos, int64_t rows, int32_t hq,
                               int32_t hkv, int32_t dh, float eps, const float* table,
                               int32_t max_pos, hipStream_t s) {
  if (dt == DFLASH_BF16) {
    if (dh == 128)
      return launch_qknr<bf16, 128>((bf16*)q, (bf16*)k, wq, wk, pos, rows, hq, hkv, eps, table,
                                    max_pos, s);
    return launch_qknr<bf16, 64>((bf16*)q, (bf16*)k, wq, wk, pos, rows, hq, hkv, eps, table,
                                 max_pos, s);
  }
  if (dh == 128)
    return launch_qknr<float, 128>((float*)q, (float*)k, wq, wk, pos, rows, hq, hkv, eps, table,
                                   max_pos, s);
  return launch_qknr<float, 64>((float*)q, (float*)k, wq, wk, pos, rows, hq, hkv, eps, table,
                                max_pos, s);
}

}  // namespace dflash
