// Device helpers shared by the libmuonh kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "desc.h"

namespace muonh {

typedef uint16_t bf16_t;  // bfloat16 storage

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// float -> bfloat16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Storage traits: load / store one element of a storage type as float.
template <typename T> struct St;
template <> struct St<float> {
  static __device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void st(float* p, int64_t i, float v) { p[i] = v; }
  static __device__ __forceinline__ float round(float v) { return v; }
  static constexpr int dt = DT_F32;
};
template <> struct St<bf16_t> {
  static __device__ __forceinline__ float ld(const bf16_t* p, int64_t i) { return bf2f(p[i]); }
  static __device__ __forceinline__ void st(bf16_t* p, int64_t i, float v) { p[i] = f2bf(v); }
  static __device__ __forceinline__ float round(float v) { return bf2f(f2bf(v)); }
  static constexpr int dt = DT_BF16;
};

// Load 8 consecutive elements [i, i+8) as float.  vec: the caller knows the
// 8 elements are in range and 16-byte (bf16) / 32-byte (f32) aligned.
__device__ __forceinline__ void load8(const bf16_t* p, int64_t i, float (&v)[8]) {
  uint4 q = *reinterpret_cast<const uint4*>(p + i);
  uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[2 * k] = __uint_as_float(w[k] << 16);
    v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, int64_t i, float (&v)[8]) {
  float4 a = *reinterpret_cast<const float4*>(p + i);
  float4 b = *reinterpret_cast<const float4*>(p + i + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void store8(bf16_t* p, int64_t i, const float (&v)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) w[k] = (uint32_t)f2bf(v[2 * k]) | ((uint32_t)f2bf(v[2 * k + 1]) << 16);
  *reinterpret_cast<uint4*>(p + i) = make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ __forceinline__ void store8(float* p, int64_t i, const float (&v)[8]) {
  *reinterpret_cast<float4*>(p + i) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + i + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// Store one element of run-time dtype.
__device__ __forceinline__ float store_dyn(void* p, int64_t i, float v, int dtype) {
  if (dtype == DT_BF16) {
    uint16_t h = f2bf(v);
    reinterpret_cast<bf16_t*>(p)[i] = h;
    return bf2f(h);
  }
  reinterpret_cast<float*>(p)[i] = v;
  return v;
}
__device__ __forceinline__ float load_dyn(const void* p, int64_t i, int dtype) {
  if (dtype == DT_BF16) return bf2f(reinterpret_cast<const bf16_t*>(p)[i]);
  return reinterpret_cast<const float*>(p)[i];
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Block-wide sum of (v0, v1); thread 0 stores the block total as partial
// `part` of reduction slot `slot`.  No fence: a later finalize kernel (a
// kernel boundary later) sums the slot's partials in a fixed order, so the
// result is bitwise reproducible.  Must be called by every thread.
template <int NT>
__device__ void block_partial2(double v0, double v1, const SlotTable& st, int slot, int part) {
  static_assert(NT % 64 == 0, "block must be whole waves");
  constexpr int NW = NT / 64;
  __shared__ double red[2][NW];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  v0 = wave_sum(v0);
  v1 = wave_sum(v1);
  if (l == 0) { red[0][w] = v0; red[1][w] = v1; }
  __syncthreads();
  if (threadIdx.x == 0) {
    double t0 = 0.0, t1 = 0.0;
#pragma unroll
    for (int i = 0; i < NW; ++i) { t0 += red[0][i]; t1 += red[1][i]; }
    const int64_t p = st.part_base[slot] + part;
    st.partials[2 * p] = t0;
    st.partials[2 * p + 1] = t1;
  }
}

}  // namespace muonh
