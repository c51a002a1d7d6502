// Device helpers shared by the libmuonh kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "desc.h"

namespace muonh {

typedef uint16_t bf16_t;  // bfloat16 storage
typedef _Float16 f16_t;   // IEEE half storage (Newton-Schulz iterates X, A, B in MUONH_NS_H16)

// Pointers taken from descriptor tables are generic; accesses through them
// compile to flat loads/stores, which count against both the vector-memory
// and the LDS wait counters.  Everything the kernels touch in HBM goes
// through these global (address space 1) views instead.
#define MUONH_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ MUONH_GLOBAL T* gmem(T* p) { return (MUONH_GLOBAL T*)p; }
template <typename T>
__device__ __forceinline__ const MUONH_GLOBAL T* gmem(const T* p) { return (const MUONH_GLOBAL T*)p; }

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// float -> bfloat16, round to nearest even (NaN stays NaN): gfx950's
// v_cvt_pk_bf16_f32 under the default round-to-nearest-even mode.
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// Two floats -> packed bf16 pair (lo in bits 0..15), one conversion.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// IEEE half <-> float: the conversion instructions round to nearest even.
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const f16x2_t v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
// The two 16-bit values of a packed pair as float (lo in bits 0..15), for
// either 16-bit storage type.
template <typename T> __device__ __forceinline__ float lo16(uint32_t w);
template <typename T> __device__ __forceinline__ float hi16(uint32_t w);
template <> __device__ __forceinline__ float lo16<bf16_t>(uint32_t w) { return __uint_as_float(w << 16); }
template <> __device__ __forceinline__ float hi16<bf16_t>(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
template <> __device__ __forceinline__ float lo16<f16_t>(uint32_t w) {
  return (float)__builtin_bit_cast(f16x2_t, w)[0];
}
template <> __device__ __forceinline__ float hi16<f16_t>(uint32_t w) {
  return (float)__builtin_bit_cast(f16x2_t, w)[1];
}
template <typename T> __device__ __forceinline__ uint32_t pack16x2(float lo, float hi);
template <> __device__ __forceinline__ uint32_t pack16x2<bf16_t>(float lo, float hi) { return pack_bf16x2(lo, hi); }
template <> __device__ __forceinline__ uint32_t pack16x2<f16_t>(float lo, float hi) { return pack_f16x2(lo, hi); }

// Storage traits: load / store one element of a storage type as float.
template <typename T> struct St;
template <> struct St<float> {
  static __device__ __forceinline__ float ld(const float* p, int64_t i) { return gmem(p)[i]; }
  static __device__ __forceinline__ void st(float* p, int64_t i, float v) { gmem(p)[i] = v; }
  static __device__ __forceinline__ float round(float v) { return v; }
  static constexpr int dt = DT_F32;
};
template <> struct St<bf16_t> {
  static __device__ __forceinline__ float ld(const bf16_t* p, int64_t i) { return bf2f(gmem(p)[i]); }
  static __device__ __forceinline__ void st(bf16_t* p, int64_t i, float v) { gmem(p)[i] = f2bf(v); }
  static __device__ __forceinline__ float round(float v) { return bf2f(f2bf(v)); }
  static constexpr int dt = DT_BF16;
};

// Native vector types for 16 / 8-byte global accesses (HIP's uint4 / float4
// classes cannot bind address-space-1 references).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Load 8 consecutive elements [i, i+8) as float.  The caller knows the 8
// elements are in range and 16-byte (bf16) / 32-byte (f32) aligned.
__device__ __forceinline__ void load8(const bf16_t* p, int64_t i, float (&v)[8]) {
  const u32x4_t q = *reinterpret_cast<const MUONH_GLOBAL u32x4_t*>(gmem(p + i));
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[2 * k] = __uint_as_float(q[k] << 16);
    v[2 * k + 1] = __uint_as_float(q[k] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, int64_t i, float (&v)[8]) {
  const f32x4_t a = *reinterpret_cast<const MUONH_GLOBAL f32x4_t*>(gmem(p + i));
  const f32x4_t b = *reinterpret_cast<const MUONH_GLOBAL f32x4_t*>(gmem(p + i + 4));
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
  v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
}
// 8 consecutive elements held in their storage form until unpacked.  A batch
// of them can be in flight before any value is used; a conversion right next
// to its load (above all inside a branch) makes the compiler wait for that
// load there, one memory round trip per chunk.
template <typename T> struct Raw8;
template <> struct Raw8<bf16_t> {
  u32x4_t q;
  __device__ __forceinline__ void load(const bf16_t* p, int64_t i) {
    q = *reinterpret_cast<const MUONH_GLOBAL u32x4_t*>(gmem(p + i));
  }
  __device__ __forceinline__ void unpack(float (&v)[8]) const {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(q[k] << 16);
      v[2 * k + 1] = __uint_as_float(q[k] & 0xffff0000u);
    }
  }
};
template <> struct Raw8<float> {
  f32x4_t a, b;
  __device__ __forceinline__ void load(const float* p, int64_t i) {
    a = *reinterpret_cast<const MUONH_GLOBAL f32x4_t*>(gmem(p + i));
    b = *reinterpret_cast<const MUONH_GLOBAL f32x4_t*>(gmem(p + i + 4));
  }
  __device__ __forceinline__ void unpack(float (&v)[8]) const {
    v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
    v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
  }
};

// 8 floats from memory the running kernel does not write, read through the
// constant address space so the loads may be issued ahead of the kernel's
// own stores (p + i 16-byte aligned).
__device__ __forceinline__ void load8_ro(const float* p, int64_t i, float (&v)[8]) {
  typedef __attribute__((address_space(4))) const f32x4_t cf4;
  const f32x4_t a = *reinterpret_cast<cf4*>(reinterpret_cast<uintptr_t>(p + i));
  const f32x4_t b = *reinterpret_cast<cf4*>(reinterpret_cast<uintptr_t>(p + i + 4));
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
  v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
}
__device__ __forceinline__ float load1_ro(const float* p, int64_t i) {
  typedef __attribute__((address_space(4))) const float cf1;
  return *reinterpret_cast<cf1*>(reinterpret_cast<uintptr_t>(p + i));
}

__device__ __forceinline__ void store8(bf16_t* p, int64_t i, const float (&v)[8]) {
  u32x4_t w;
#pragma unroll
  for (int k = 0; k < 4; ++k) w[k] = pack_bf16x2(v[2 * k], v[2 * k + 1]);
  *reinterpret_cast<MUONH_GLOBAL u32x4_t*>(gmem(p + i)) = w;
}
__device__ __forceinline__ void store8(f16_t* p, int64_t i, const float (&v)[8]) {
  u32x4_t w;
#pragma unroll
  for (int k = 0; k < 4; ++k) w[k] = pack_f16x2(v[2 * k], v[2 * k + 1]);
  *reinterpret_cast<MUONH_GLOBAL u32x4_t*>(gmem(p + i)) = w;
}
__device__ __forceinline__ void store8(float* p, int64_t i, const float (&v)[8]) {
  const f32x4_t a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
  *reinterpret_cast<MUONH_GLOBAL f32x4_t*>(gmem(p + i)) = a;
  *reinterpret_cast<MUONH_GLOBAL f32x4_t*>(gmem(p + i + 4)) = b;
}

// Store one element of run-time dtype.
__device__ __forceinline__ float store_dyn(void* p, int64_t i, float v, int dtype) {
  if (dtype == DT_BF16) {
    uint16_t h = f2bf(v);
    gmem(reinterpret_cast<bf16_t*>(p))[i] = h;
    return bf2f(h);
  }
  gmem(reinterpret_cast<float*>(p))[i] = v;
  return v;
}
__device__ __forceinline__ float load_dyn(const void* p, int64_t i, int dtype) {
  if (dtype == DT_BF16) return bf2f(gmem(reinterpret_cast<const bf16_t*>(p))[i]);
  return gmem(reinterpret_cast<const float*>(p))[i];
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
// block_partial2_at takes its LDS scratch (2 NT / 64 doubles) from the
// caller; block_partial2 uses a static array of its own.
template <int NT>
__device__ void block_partial2_at(double v0, double v1, const SlotTable& st, int slot, int part,
                                  double (*red)[NT / 64]) {
  static_assert(NT % 64 == 0, "block must be whole waves");
  constexpr int NW = NT / 64;
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
    gmem(st.partials)[2 * p] = t0;
    gmem(st.partials)[2 * p + 1] = t1;
  }
}
template <int NT>
__device__ void block_partial2(double v0, double v1, const SlotTable& st, int slot, int part) {
  __shared__ double red[2][NT / 64];
  block_partial2_at<NT>(v0, v1, st, slot, part, red);
}

// Three per-block sums: (a, b) into slot_a, (0, c) into slot_b, both at
// partial index part (one shared-memory round, deterministic order).
template <int NT>
__device__ void block_partial3(double a, double b, double c, const SlotTable& st, int slot_a, int slot_b, int part) {
  static_assert(NT % 64 == 0, "block must be whole waves");
  constexpr int NW = NT / 64;
  __shared__ double red3[3][NW];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  a = wave_sum(a);
  b = wave_sum(b);
  c = wave_sum(c);
  if (l == 0) { red3[0][w] = a; red3[1][w] = b; red3[2][w] = c; }
  __syncthreads();
  if (threadIdx.x == 0) {
    double t0 = 0.0, t1 = 0.0, t2 = 0.0;
#pragma unroll
    for (int i = 0; i < NW; ++i) { t0 += red3[0][i]; t1 += red3[1][i]; t2 += red3[2][i]; }
    const int64_t pa = st.part_base[slot_a] + part, pb = st.part_base[slot_b] + part;
    gmem(st.partials)[2 * pa] = t0;
    gmem(st.partials)[2 * pa + 1] = t1;
    gmem(st.partials)[2 * pb] = 0.0;
    gmem(st.partials)[2 * pb + 1] = t2;
  }
}

}  // namespace muonh
