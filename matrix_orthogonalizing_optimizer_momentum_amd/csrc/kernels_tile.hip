// Resident-tile Newton-Schulz for Hierarchical Muon (gfx950).
//
// "Hierarchical Muon: Tiled Newton-Schulz Updates for Efficient Muon
// Optimization" (core claim, abstract): each momentum matrix is cut into
// T x T tiles from (0, 0) and the same finite Newton-Schulz map runs on every
// tile on its own.  For T <= 128 one workgroup owns one tile for the whole
// step:
//   - momentum M <- beta M + G for the tile's elements (Muon explainer,
//     momentum recap / Equation 1), stored back, or the plain NS input;
//   - the tile zero-padded to TP x TP (TP = 64 or 128; zero padding is exact:
//     [[X, 0], [0, 0]] maps to [[NS(X), 0], [0, 0]]) and its own Frobenius
//     norm, with 1 / (||X0|| + eps) folded into the first iteration;
//   - K iterations A = X X^T; B = b A + c A A; X = a X + B X (Muon explainer,
//     Equation 6 and code section) out of LDS, with the fp32 master X held in
//     the MFMA accumulator layout in registers;
//   - the cropped tile written once, with its sum of squares as one partial of
//     the matrix's ||O||^2 for the Hyperball normalization.
// Nothing but the tile's inputs and output touches HBM.
//
// LDS (bf16 operands): sX holds X row-major for A = X X^T, sT holds X^T for
// B X; A and then B overwrite sX once A has been formed (X is needed again
// only after the update, and X^T and the fp32 master still hold it).  Both A
// and B are symmetric, so they are stored through the transposed (packed)
// path.  fp32 operands read X column-wise instead of keeping X^T, so A and B
// take a buffer of their own.
#include "common.h"

namespace muonh {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

constexpr int kTileThreads = 256;

template <typename T> struct TileOp;
template <> struct TileOp<bf16_t> {
  static constexpr int KSTEP = 16;
  static constexpr int PAD = 8;  // 16 bytes: conflict-free 16-byte fragment reads
  static __device__ __forceinline__ void put(bf16_t* p, float v) { *p = f2bf(v); }
  // p[0..3] = v0..v3; p is 8-byte aligned
  static __device__ __forceinline__ void put4(bf16_t* p, float v0, float v1, float v2, float v3) {
    u32x2_t w;
    w[0] = (uint32_t)f2bf(v0) | ((uint32_t)f2bf(v1) << 16);
    w[1] = (uint32_t)f2bf(v2) | ((uint32_t)f2bf(v3) << 16);
    *reinterpret_cast<u32x2_t*>(p) = w;
  }
  static __device__ __forceinline__ void get4(const bf16_t* p, float (&v)[4]) {
    const u32x2_t w = *reinterpret_cast<const u32x2_t*>(p);
    v[0] = __uint_as_float(w[0] << 16);
    v[1] = __uint_as_float(w[0] & 0xffff0000u);
    v[2] = __uint_as_float(w[1] << 16);
    v[3] = __uint_as_float(w[1] & 0xffff0000u);
  }
};
template <> struct TileOp<float> {
  static constexpr int KSTEP = 2;
  static constexpr int PAD = 2;
  static __device__ __forceinline__ void put(float* p, float v) { *p = v; }
  static __device__ __forceinline__ void put4(float* p, float v0, float v1, float v2, float v3) {
    u32x2_t a, b;  // 8-byte aligned (even pitch, rows in fours)
    a[0] = __float_as_uint(v0); a[1] = __float_as_uint(v1);
    b[0] = __float_as_uint(v2); b[1] = __float_as_uint(v3);
    reinterpret_cast<u32x2_t*>(p)[0] = a;
    reinterpret_cast<u32x2_t*>(p)[1] = b;
  }
  static __device__ __forceinline__ void get4(const float* p, float (&v)[4]) {
    v[0] = p[0]; v[1] = p[1]; v[2] = p[2]; v[3] = p[3];
  }
};

// Accumulator layout of v_mfma_f32_32x32x* (wave64): register v of a 32 x 32
// block holds row 8*(v/4) + 4*(lane/32) + v%4, column lane%32.
__device__ __forceinline__ int acc_row(int v, int lane) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }

}  // namespace

// TP: padded tile side (64 or 128).  ST: momentum / input storage type,
// OT: Newton-Schulz operand type.
template <typename ST, typename OT, int TP>
__global__ __launch_bounds__(kTileThreads) __attribute__((amdgpu_waves_per_eu(2))) void k_tile_ns(const TileMat* __restrict__ mats,
                                                          const TileJob* __restrict__ jobs, TileArgs args) {
  using Op = TileOp<OT>;
  constexpr int LD = TP + Op::PAD;           // LDS pitch (elements)
  constexpr int WT = TP / 2;                 // wave tile side (2 x 2 waves)
  constexpr int MI = WT / 32;                // 32 x 32 accumulator blocks per wave side
  constexpr bool kXT = sizeof(OT) == 2;      // bf16: keep X^T for B X
  __shared__ __attribute__((aligned(16))) OT sX[TP * LD];
  __shared__ __attribute__((aligned(16))) OT sT[TP * LD];  // bf16: X^T; fp32: A, then B
  __shared__ double sred[4];
  __shared__ float ssig;
  OT* const sAB = kXT ? sX : sT;

  const TileJob job = jobs[blockIdx.x];
  const TileMat mt = mats[job.mat];
  const int T = args.T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = (wave >> 1) * WT, wc = (wave & 1) * WT;  // wave tile origin
  const int lc = lane & 31;
  const int64_t r0 = (int64_t)job.ti * T, c0 = (int64_t)job.tj * T;
  const int h = (int)min<int64_t>(T, mt.H - r0), w = (int)min<int64_t>(T, mt.W - c0);
  const ST* __restrict__ gp = reinterpret_cast<const ST*>(mt.g);
  ST* __restrict__ mp = reinterpret_cast<ST*>(mt.m);

  // ---- tile load (+ momentum), in the accumulator layout: every thread owns
  // the same elements from here to the final store.
  float x32[MI][MI][16];
  float sq = 0.f;
  const ST* tg = gp ? gp + r0 * mt.W + c0 : nullptr;
  ST* tm = mp + r0 * mt.W + c0;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    float mv[MI][16], gv[MI][16];
#pragma unroll
    for (int j = 0; j < MI; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wr + i * 32 + acc_row(v, lane), col = wc + j * 32 + lc;
        // clamped to the tile origin outside the matrix: always in bounds
        const int64_t o = (row < h && col < w) ? (int64_t)row * mt.W + col : 0;
        mv[j][v] = St<ST>::ld(tm, o);
        gv[j][v] = tg ? St<ST>::ld(tg, o) : 0.f;
      }
#pragma unroll
    for (int j = 0; j < MI; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wr + i * 32 + acc_row(v, lane), col = wc + j * 32 + lc;
        const bool ok = row < h && col < w;
        float x = mv[j][v];
        if (tg) {
          x = St<ST>::round(fmaf(args.beta, x, gv[j][v]));
          if (ok) St<ST>::st(tm, (int64_t)row * mt.W + col, x);
        }
        x = ok ? x : 0.f;
        sq = fmaf(x, x, sq);
        x32[i][j][v] = args.fold ? bf2f(f2bf(x)) : x;  // fold: X itself is kept in bf16
      }
  }
  // X0 into LDS (unscaled): sX row-major, and sT = X^T for bf16 operands.
  auto store_x = [&]() {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < MI; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = wr + i * 32 + acc_row(4 * q, lane), col = wc + j * 32 + lc;
#pragma unroll
          for (int e = 0; e < 4; ++e) Op::put(&sX[(row + e) * LD + col], x32[i][j][4 * q + e]);
          if (kXT)
            Op::put4(&sT[col * LD + row], x32[i][j][4 * q], x32[i][j][4 * q + 1], x32[i][j][4 * q + 2],
                     x32[i][j][4 * q + 3]);
        }
  };
  store_x();
  {
    const double d = wave_sum((double)sq);
    if (lane == 0) sred[wave] = d;
    __syncthreads();
    if (tid == 0) ssig = (float)(1.0 / (sqrt(((sred[0] + sred[1]) + sred[2]) + sred[3]) + (double)args.eps));
    __syncthreads();
  }
  const double sig = (double)ssig;

  f32x16_t acc[MI][MI];
  // acc += P Q^T over k in [0, TP): P rows from sp (row-major, k contiguous);
  // Q rows from sq (k contiguous) or, with q_kn, Q(n, k) = sq[k][n].
  auto product = [&](const OT* sp, const OT* sq_, bool q_kn) {
#pragma unroll 2
    for (int k = 0; k < TP; k += Op::KSTEP) {
      const int kk = k + (lane >> 5) * (Op::KSTEP / 2);
      if constexpr (sizeof(OT) == 2) {
        bf16x8_t fa[MI], fb[MI];
#pragma unroll
        for (int i = 0; i < MI; ++i) fa[i] = *reinterpret_cast<const bf16x8_t*>(sp + (wr + i * 32 + lc) * LD + kk);
#pragma unroll
        for (int j = 0; j < MI; ++j) fb[j] = *reinterpret_cast<const bf16x8_t*>(sq_ + (wc + j * 32 + lc) * LD + kk);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < MI; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      } else {
        float fa[MI], fb[MI];
#pragma unroll
        for (int i = 0; i < MI; ++i) fa[i] = sp[(wr + i * 32 + lc) * LD + kk];
#pragma unroll
        for (int j = 0; j < MI; ++j)
          fb[j] = q_kn ? sq_[kk * LD + wc + j * 32 + lc] : sq_[(wc + j * 32 + lc) * LD + kk];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < MI; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i], fb[j], acc[i][j], 0, 0, 0);
      }
    }
  };
  // Symmetric result (A or B) = acc * sc into sAB through the packed
  // transposed path: sAB[col][row .. row+3].
  auto store_sym = [&](float sc) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < MI; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = wr + i * 32 + acc_row(4 * q, lane), col = wc + j * 32 + lc;
          Op::put4(&sAB[col * LD + row], acc[i][j][4 * q] * sc, acc[i][j][4 * q + 1] * sc,
                   acc[i][j][4 * q + 2] * sc, acc[i][j][4 * q + 3] * sc);
        }
  };

  for (int it = 0; it < args.K; ++it) {
    const float a = args.abc[it][0], b = args.abc[it][1], c = args.abc[it][2];
    const bool first = it == 0;
    // G1: A = X X^T (times sig^2 on the first iteration: X0 is unscaled)
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < MI; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    product(sX, sX, false);
    __syncthreads();  // bf16: every wave is done reading X before A overwrites it
    store_sym(first ? (float)(sig * sig) : 1.f);
    __syncthreads();
    // G2: B = b A + c A A, as c (A A + (b/c) A) with the accumulator seeded
    // from A; c == 0 leaves B = b A.
    {
      const float seed = c != 0.f ? b / c : b;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < MI; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int row = wr + i * 32 + acc_row(4 * q, lane), col = wc + j * 32 + lc;
            float av[4];
            Op::get4(&sAB[col * LD + row], av);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][4 * q + e] = seed * av[e];
          }
    }
    if (c != 0.f) product(sAB, sAB, false);
    __syncthreads();  // every wave is done reading A
    store_sym(c != 0.f ? c : 1.f);
    __syncthreads();
    // G3: X <- a X + B X, seeded with a X from the fp32 master
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < MI; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = a * x32[i][j][v];
    if constexpr (kXT) product(sAB, sT, false);
    else product(sAB, sX, true);
    __syncthreads();  // every wave is done reading B, X and X^T
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < MI; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float t = acc[i][j][v];
          if (first) t = (float)((double)t * sig);
          if (args.fold) t = bf2f(f2bf(t));
          x32[i][j][v] = t;
        }
    if (it + 1 < args.K) {
      store_x();
      __syncthreads();
    }
  }
  if (args.K == 0) {  // O = X0 / (||X0|| + eps)
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < MI; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) x32[i][j][v] = (float)((double)x32[i][j][v] * sig);
  }

  // ---- cropped tile out, sum of squares of the stored values
  float osq = 0.f;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < MI; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wr + i * 32 + acc_row(v, lane), col = wc + j * 32 + lc;
        if (row < h && col < w) {
          const float s = store_dyn(mt.out, (r0 + row) * mt.W + c0 + col, x32[i][j][v], mt.out_dtype);
          osq = fmaf(s, s, osq);
        }
      }
  block_partial2<kTileThreads>((double)osq, 0.0, args.st, mt.onorm_slot, job.part);
}

namespace {
template <typename ST, typename OT>
void launch_tile_t(int TP, dim3 grid, const TileMat* mats, const TileJob* jobs, const TileArgs& args, hipStream_t s) {
  if (TP == 64) hipLaunchKernelGGL((k_tile_ns<ST, OT, 64>), grid, dim3(kTileThreads), 0, s, mats, jobs, args);
  else hipLaunchKernelGGL((k_tile_ns<ST, OT, 128>), grid, dim3(kTileThreads), 0, s, mats, jobs, args);
}
}  // namespace

hipError_t launch_tile_ns(int state_dt, int op_dt, const TileMat* mats, const TileJob* jobs, int njobs,
                          const TileArgs& args, hipStream_t s) {
  if (njobs <= 0) return hipSuccess;
  if (args.T < 1 || args.T > kTileResidentMax || args.K < 0 || args.K > kTileMaxK) return hipErrorInvalidValue;
  const int TP = args.T <= 64 ? 64 : 128;
  const dim3 grid(njobs);
  if (state_dt == DT_BF16 && op_dt == DT_BF16) launch_tile_t<bf16_t, bf16_t>(TP, grid, mats, jobs, args, s);
  else if (state_dt == DT_BF16) launch_tile_t<bf16_t, float>(TP, grid, mats, jobs, args, s);
  else if (op_dt == DT_BF16) launch_tile_t<float, bf16_t>(TP, grid, mats, jobs, args, s);
  else launch_tile_t<float, float>(TP, grid, mats, jobs, args, s);
  return hipGetLastError();
}

}  // namespace muonh
