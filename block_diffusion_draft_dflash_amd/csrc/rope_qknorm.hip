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

template <typename T>
struct Vec4;
template <>
struct Vec4<bf16> {
  typedef bf16x4 type;
  static __device__ __forceinline__ void load(const bf16* p, float* x) {
    bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = bf2f(v[e]);
  }
  static __device__ __forceinline__ void store(bf16* p, const float* x) {
    bf16x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = f2bf(x[e]);
    *reinterpret_cast<bf16x4*>(p) = v;
  }
};
template <>
struct Vec4<float> {
  static __device__ __forceinline__ void load(const float* p, float* x) {
    float4 v = *reinterpret_cast<const float4*>(p);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
  }
  static __device__ __forceinline__ void store(float* p, const float* x) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  }
};

// One head vector per group of DH/8 lanes. Lane s of the group holds elements
// [4s, 4s+4) of the first half and their rotation partners [DH/2+4s, DH/2+4s+4).
template <typename T, int DH>
__global__ __launch_bounds__(256) void qk_norm_rope_kernel(
    T* __restrict__ q, T* __restrict__ k, const float* __restrict__ wq,
    const float* __restrict__ wk, const int32_t* __restrict__ pos,
    const float2* __restrict__ table, int32_t max_pos, int64_t rows, int32_t hq, int32_t hkv,
    float eps) {
  // every argument in one batch of scalar loads (no dependent argument reads)
  asm volatile("" ::"s"(q), "s"(k), "s"(wq), "s"(wk), "s"(pos), "s"(table), "s"(max_pos), "s"(rows),
               "s"(hq), "s"(hkv), "s"(eps));
  constexpr int LANES = DH / 8;
  constexpr int PER_WAVE = 64 / LANES;
  constexpr int HALF = DH / 2;
  const int lane = threadIdx.x & 63;
  const int s = lane % LANES;
  const int64_t vec = ((int64_t)blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64) * PER_WAVE +
                      lane / LANES;
  const int32_t hq_eff = q ? hq : 0;
  const int32_t heads = hq_eff + hkv;
  const bool valid = vec < rows * heads;
  const int64_t row = valid ? vec / heads : 0;
  const int32_t h = valid ? (int32_t)(vec % heads) : 0;
  T* base = (h < hq_eff) ? q + (row * hq + h) * DH : k + (row * hkv + (h - hq_eff)) * DH;
  const float* w = (h < hq_eff) ? wq : wk;

  float x0[4] = {0.f, 0.f, 0.f, 0.f}, x1[4] = {0.f, 0.f, 0.f, 0.f};
  if (valid) {
    Vec4<T>::load(base + 4 * s, x0);
    Vec4<T>::load(base + HALF + 4 * s, x1);
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) ss += x0[e] * x0[e] + x1[e] * x1[e];
  ss = group_sum<LANES>(ss);  // all lanes of a group share `valid`
  const float inv = 1.0f / sqrtf(ss * (1.0f / DH) + eps);
  if (!valid) return;
  int32_t p = pos[row];
  p = p < 0 ? 0 : (p >= max_pos ? max_pos - 1 : p);
  const float4* cs4 = reinterpret_cast<const float4*>(table + (int64_t)p * HALF + 4 * s);
  const float4 c01 = cs4[0], c23 = cs4[1];
  const float cs[8] = {c01.x, c01.y, c01.z, c01.w, c23.x, c23.y, c23.z, c23.w};
  const float4 w0 = *reinterpret_cast<const float4*>(w + 4 * s);
  const float4 w1 = *reinterpret_cast<const float4*>(w + HALF + 4 * s);
  const float wa[4] = {w0.x, w0.y, w0.z, w0.w}, wb[4] = {w1.x, w1.y, w1.z, w1.w};
  float y0[4], y1[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a = x0[e] * inv * wa[e];
    const float b = x1[e] * inv * wb[e];
    const float c = cs[2 * e], sn = cs[2 * e + 1];
    y0[e] = a * c - b * sn;
    y1[e] = b * c + a * sn;
  }
  Vec4<T>::store(base + 4 * s, y0);
  Vec4<T>::store(base + HALF + 4 * s, y1);
}

template <typename T, int DH>
hipError_t launch_qknr(T* q, T* k, const float* wq, const float* wk, const int32_t* pos,
                       int64_t rows, int32_t hq, int32_t hkv, float eps, const float* table,
                       int32_t max_pos, hipStream_t s) {
  const int64_t heads = (q ? hq : 0) + hkv;
  const int64_t vecs = rows * heads;
  const int64_t per_block = 4 * (64 / (DH / 8));
  const int64_t blocks = (vecs + per_block - 1) / per_block;
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
