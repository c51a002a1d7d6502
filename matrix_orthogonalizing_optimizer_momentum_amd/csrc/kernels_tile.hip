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
#include <type_traits>

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
  // p[0] = v0, p[ld] = v1 (two rows of one column, one conversion)
  static __device__ __forceinline__ void put2col(bf16_t* p, int ld, float v0, float v1) {
    const uint32_t w = pack_bf16x2(v0, v1);
    p[0] = (bf16_t)w;
    p[ld] = (bf16_t)(w >> 16);
  }
  // p[0..3] = v0..v3; p is 8-byte aligned
  static __device__ __forceinline__ void put4(bf16_t* p, float v0, float v1, float v2, float v3) {
    const u32x2_t w = {pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
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
  static __device__ __forceinline__ void put2col(float* p, int ld, float v0, float v1) {
    p[0] = v0;
    p[ld] = v1;
  }
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
// OT: Newton-Schulz operand type; FOLD: X rounded to bf16 after every update
// (bf16 operands without the fp32 master copy).  With bf16 operands two workgroups fit one
// CU's LDS, so registers are capped for two waves per SIMD; a 128-side fp32
// tile takes most of the LDS on its own.
template <typename ST, typename OT, int TP, bool FOLD>
__global__ __launch_bounds__(kTileThreads) __attribute__((amdgpu_waves_per_eu(sizeof(OT) == 2 ? 2 : 1)))
void k_tile_ns(const TileMat* __restrict__ mats, const TileJob* __restrict__ jobs, TileArgs args) {
  using Op = TileOp<OT>;
  constexpr int LD = TP + Op::PAD;           // LDS pitch (elements)
  constexpr int WT = TP / 2;                 // wave tile side (2 x 2 waves)
  constexpr int MI = WT / 32;                // 32 x 32 accumulator blocks per wave side
  constexpr bool kXT = sizeof(OT) == 2;      // bf16: keep X^T for B X
  // One LDS block: sX, sT (bf16: X^T; fp32: A, then B) and, aliasing both,
  // an fp32 staging tile for the coalesced load and store phases.
  constexpr int XB = TP * LD * (int)sizeof(OT);
  constexpr int SP = TP + 4;                 // staging pitch (floats)
  constexpr int kSmem = 2 * XB > TP * SP * 4 ? 2 * XB : TP * SP * 4;
  __shared__ __attribute__((aligned(16))) char smem[kSmem];
  __shared__ double sred[4];
  __shared__ float ssig;
  OT* const sX = reinterpret_cast<OT*>(smem);
  OT* const sT = reinterpret_cast<OT*>(smem + XB);
  float* const stg = reinterpret_cast<float*>(smem);
  OT* const sAB = kXT ? sX : sT;

  const TileJob job = jobs[blockIdx.x];
  const TileMat mt = mats[job.mat];
  const int T = args.T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = (wave >> 1) * WT, wc = (wave & 1) * WT;  // wave tile origin
  const int lc = lane & 31;
  const int64_t r0 = (int64_t)job.ti * T, c0 = (int64_t)job.tj * T;
  const int h = (int)min<int64_t>(T, mt.H - r0), w = (int)min<int64_t>(T, mt.W - c0);
  const int64_t ldm = mt.W;
  const ST* tg = mt.g ? reinterpret_cast<const ST*>(mt.g) + r0 * ldm + c0 : nullptr;
  ST* tm = reinterpret_cast<ST*>(mt.m) + r0 * ldm + c0;

  // ---- load phase: the tile in 8-element row chunks (thread t takes chunks
  // t, t + 256, ...: consecutive threads read consecutive 16-byte pieces),
  // momentum, M stored back, fp32 values staged row-major in LDS.
  constexpr int CPR = TP / 8;                // chunks per row
  constexpr int NCH = TP * CPR / kTileThreads;  // chunks per thread
  static_assert(NCH * kTileThreads == TP * CPR, "whole chunks per thread");
  float sq = 0.f;
  if (mt.vec) {
    // Whole chunks are either inside the matrix or outside it (8-aligned
    // sides and origins); outside ones load the tile origin's chunk instead
    // (always valid) and are zeroed.  Every chunk's loads are issued before
    // any is converted.
    Raw8<ST> mr[NCH], gr[NCH];
    auto chunk_off = [&](int c) -> int64_t {
      const int ch = tid + c * kTileThreads, row = ch / CPR, col = (ch % CPR) * 8;
      return (row < h && col < w) ? (int64_t)row * ldm + col : 0;
    };
#pragma unroll
    for (int c = 0; c < NCH; ++c) mr[c].load(tm, chunk_off(c));
    if (tg) {
#pragma unroll
      for (int c = 0; c < NCH; ++c) gr[c].load(tg, chunk_off(c));
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int ch = tid + c * kTileThreads, row = ch / CPR, col = (ch % CPR) * 8;
      const bool ok = row < h && col < w;
      float x[8];
      mr[c].unpack(x);
      if (tg) {
        float gv[8];
        gr[c].unpack(gv);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = St<ST>::round(fmaf(args.beta, x[e], args.gcoef * gv[e]));
        if (ok) store8(tm, (int64_t)row * ldm + col, x);
        if (args.nesterov) {  // NS input: the Nesterov blend of G and the updated buffer
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = fmaf(args.beta, x[e], args.gcoef * gv[e]);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = ok ? x[e] : 0.f;
        sq = fmaf(x[e], x[e], sq);
      }
      f32x4_t* d = reinterpret_cast<f32x4_t*>(stg + row * SP + col);
      d[0] = f32x4_t{x[0], x[1], x[2], x[3]};
      d[1] = f32x4_t{x[4], x[5], x[6], x[7]};
    }
  } else {
#pragma unroll 1
    for (int c = 0; c < NCH; ++c) {
      const int ch = tid + c * kTileThreads, row = ch / CPR, col = (ch % CPR) * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x = 0.f;
        if (row < h && col + e < w) {
          const int64_t o = (int64_t)row * ldm + col + e;
          x = St<ST>::ld(tm, o);
          if (tg) {
            const float gg = St<ST>::ld(tg, o);
            x = St<ST>::round(fmaf(args.beta, x, args.gcoef * gg));
            St<ST>::st(tm, o, x);
            if (args.nesterov) x = fmaf(args.beta, x, args.gcoef * gg);
          }
        }
        sq = fmaf(x, x, sq);
        stg[row * SP + col + e] = x;
      }
    }
  }
  {
    const double d = wave_sum((double)sq);
    if (lane == 0) sred[wave] = d;
  }
  __syncthreads();
  if (tid == 0) ssig = (float)(1.0 / (sqrt(((sred[0] + sred[1]) + sred[2]) + sred[3]) + (double)args.eps));
  // Every thread takes its elements in the accumulator layout, which it owns
  // from here to the final store.  X0 is kept as formed (fp32): when it is
  // not a bf16 value (fp32 state, or the Nesterov blend) the first a X term
  // uses it unrounded; the operand copies below are rounded, and with fold
  // every later X is rounded to bf16 after its update.
  float x32[MI][MI][16];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < MI; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) x32[i][j][v] = stg[(wr + i * 32 + acc_row(v, lane)) * SP + wc + j * 32 + lc];
  __syncthreads();  // staging is overwritten by the operand copies below
  // X0 into LDS (unscaled): sX row-major, and sT = X^T for bf16 operands.
  auto store_x = [&]() {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < MI; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = wr + i * 32 + acc_row(4 * q, lane), col = wc + j * 32 + lc;
          Op::put2col(&sX[row * LD + col], LD, x32[i][j][4 * q], x32[i][j][4 * q + 1]);
          Op::put2col(&sX[(row + 2) * LD + col], LD, x32[i][j][4 * q + 2], x32[i][j][4 * q + 3]);
          if (kXT)
            Op::put4(&sT[col * LD + row], x32[i][j][4 * q], x32[i][j][4 * q + 1], x32[i][j][4 * q + 2],
                     x32[i][j][4 * q + 3]);
        }
  };
  store_x();
  __syncthreads();
  const double sig = (double)ssig;

  f32x16_t acc[MI][MI];
  // acc += P Q^T over k in [0, TP): P rows from sp (row-major, k contiguous);
  // Q rows from sq (k contiguous) or, with q_kn, Q(n, k) = sq[k][n].
  // Fragments of k-step ks are loaded one step ahead of the MFMAs that use
  // them (register double buffer); scheduling barriers keep the compiler from
  // sinking the loads next to their uses.
  constexpr int NK = TP / Op::KSTEP;
  static_assert(NK % 2 == 0, "k-steps come in pairs");
  using Frag = typename std::conditional<sizeof(OT) == 2, bf16x8_t, float>::type;
  // The first k-step takes a zero C operand (the accumulators need no
  // clearing), so a product starts from zero.
  auto product = [&](const OT* sp, const OT* sq_, bool q_kn) {
    const int kl = (lane >> 5) * (Op::KSTEP / 2);
    const OT* pa = sp + (wr + lc) * LD + kl;
    const OT* pb = sq_ + (wc + lc) * LD + kl;
    const OT* pt = sq_ + kl * LD + wc + lc;  // q_kn (fp32 only)
    Frag fa[2][MI], fb[2][MI];
    auto load = [&](int buf, int ks) {
      const int k = ks * Op::KSTEP;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        if constexpr (sizeof(OT) == 2) fa[buf][i] = *reinterpret_cast<const bf16x8_t*>(pa + i * 32 * LD + k);
        else fa[buf][i] = pa[i * 32 * LD + k];
      }
#pragma unroll
      for (int j = 0; j < MI; ++j) {
        if constexpr (sizeof(OT) == 2) fb[buf][j] = *reinterpret_cast<const bf16x8_t*>(pb + j * 32 * LD + k);
        else fb[buf][j] = q_kn ? pt[k * LD + j * 32] : pb[j * 32 * LD + k];
      }
    };
    auto mma = [&](int buf, auto zc) {
      constexpr bool zero = decltype(zc)::value;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < MI; ++j) {
          const f32x16_t c_in = zero ? f32x16_t{} : acc[i][j];
          if constexpr (sizeof(OT) == 2)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j], c_in, 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[buf][i], fb[buf][j], c_in, 0, 0, 0);
        }
    };
    load(0, 0);
    load(1, 1);
    __builtin_amdgcn_sched_barrier(0);
    mma(0, std::true_type{});
    __builtin_amdgcn_sched_barrier(0);
    load(0, min(2, NK - 1));
    __builtin_amdgcn_sched_barrier(0);
    mma(1, std::false_type{});
    __builtin_amdgcn_sched_barrier(0);
    constexpr int kUnroll = sizeof(OT) == 2 ? NK / 2 : 4;
#pragma unroll kUnroll
    for (int ks = 2; ks < NK; ks += 2) {
      load(1, ks + 1);
      __builtin_amdgcn_sched_barrier(0);
      mma(0, std::false_type{});
      __builtin_amdgcn_sched_barrier(0);
      load(0, min(ks + 2, NK - 1));  // the last one re-reads a valid step, unused
      __builtin_amdgcn_sched_barrier(0);
      mma(1, std::false_type{});
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Symmetric result (A, times sc when scaled) into sAB through the packed
  // transposed path: sAB[col][row .. row+3].
  auto store_a = [&](auto scaled, float sc) {
    constexpr bool kScale = decltype(scaled)::value;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < MI; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = wr + i * 32 + acc_row(4 * q, lane), col = wc + j * 32 + lc;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = kScale ? acc[i][j][4 * q + e] * sc : acc[i][j][4 * q + e];
          Op::put4(&sAB[col * LD + row], v[0], v[1], v[2], v[3]);
        }
  };
  // B = c A A + b A in place of A: each lane reads back the A values at the
  // very positions it then overwrites (c A A is in the accumulators).
  auto store_b = [&](float b, float c) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < MI; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = wr + i * 32 + acc_row(4 * q, lane), col = wc + j * 32 + lc;
          float av[4], v[4];
          Op::get4(&sAB[col * LD + row], av);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = fmaf(c, acc[i][j][4 * q + e], b * av[e]);
          Op::put4(&sAB[col * LD + row], v[0], v[1], v[2], v[3]);
        }
  };

  // One iteration; the first (FIRST) folds the pre-scale: A = sig^2 X0 X0^T
  // and X1 = sig (a X0 + B X0).  It is instantiated apart from the others, so
  // the later iterations carry no scale factors or run-time selects.
  auto iterate = [&](auto first_c, int it) {
    constexpr bool FIRST = decltype(first_c)::value;
    const float a = args.abc[it][0], b = args.abc[it][1], c = args.abc[it][2];
    // G1: A = X X^T
    product(sX, sX, false);
    __syncthreads();  // bf16: every wave is done reading X before A overwrites it
    store_a(std::integral_constant<bool, FIRST>{}, (float)(sig * sig));
    __syncthreads();
    // G2: B = b A + c A A (c == 0: B = b A, no product)
    if (c != 0.f) {
      product(sAB, sAB, false);
    } else {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < MI; ++j) acc[i][j] = f32x16_t{};
    }
    __syncthreads();  // every wave is done reading A
    store_b(b, c);
    __syncthreads();
    // G3: B X; the update adds a X from the fp32 master
    if constexpr (kXT) product(sAB, sT, false);
    else product(sAB, sX, true);
    __syncthreads();  // every wave is done reading B, X and X^T
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < MI; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float t = fmaf(a, x32[i][j][v], acc[i][j][v]);
          if constexpr (FIRST) t = (float)((double)t * sig);
          if constexpr (FOLD) t = bf2f(f2bf(t));
          x32[i][j][v] = t;
        }
    if (it + 1 < args.K) {
      store_x();
      __syncthreads();
    }
  };
  if (args.K > 0) {
    iterate(std::true_type{}, 0);
    for (int it = 1; it < args.K; ++it) iterate(std::false_type{}, it);
  }
  if (args.K == 0) {  // O = X0 / (||X0|| + eps)
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < MI; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) x32[i][j][v] = (float)((double)x32[i][j][v] * sig);
  }

  // ---- store phase: the result staged row-major in LDS (the last update's
  // operand reads are behind a barrier), then written as 8-element chunks,
  // cropped to the matrix; sum of squares of the stored values.  The weight
  // rows the hook's sums need do not depend on the result: their loads are
  // issued first.
  const float* const wp = mt.w;
  const int64_t obase = r0 * ldm + c0;
  typedef __attribute__((address_space(4))) const f32x4_t cf4;
  f32x4_t wv[NCH][2];
  const bool wvec = mt.vec && wp != nullptr;
  if (wvec) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int ch = tid + c * kTileThreads, row = ch / CPR, col = (ch % CPR) * 8;
      const int64_t o = (row < h && col < w) ? obase + (int64_t)row * ldm + col : obase;
      wv[c][0] = *reinterpret_cast<cf4*>(reinterpret_cast<uintptr_t>(wp + o));
      wv[c][1] = *reinterpret_cast<cf4*>(reinterpret_cast<uintptr_t>(wp + o + 4));
    }
  }
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < MI; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) stg[(wr + i * 32 + acc_row(v, lane)) * SP + wc + j * 32 + lc] = x32[i][j][v];
  __syncthreads();
  // ||O||^2 of the stored values and, for the weight-update hook, <W, O> and
  // ||W||^2 at the same positions (fp64 per thread: the hook forms
  // ||W - c O||^2 from them, which must resolve an exactly cancelling step).
  double osq = 0.0, swo = 0.0, sww = 0.0;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int ch = tid + c * kTileThreads, row = ch / CPR, col = (ch % CPR) * 8;
    if (row >= h || col >= w) continue;
    const f32x4_t* sp = reinterpret_cast<const f32x4_t*>(stg + row * SP + col);
    const f32x4_t lo = sp[0], hi = sp[1];
    float x[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    const int64_t o = obase + (int64_t)row * ldm + col;
    if (mt.out_dtype == DT_BF16) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = bf2f(f2bf(x[e]));
    }
    if (mt.vec) {
      if (mt.out_dtype == DT_BF16) store8(reinterpret_cast<bf16_t*>(mt.out), o, x);
      else store8(reinterpret_cast<float*>(mt.out), o, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) osq = fma((double)x[e], (double)x[e], osq);
      if (wvec) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double wd = (double)wv[c][e >> 2][e & 3];
          swo = fma(wd, (double)x[e], swo);
          sww = fma(wd, wd, sww);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (col + e < w) {
          store_dyn(mt.out, o + e, x[e], mt.out_dtype);
          osq = fma((double)x[e], (double)x[e], osq);
          if (wp != nullptr) {
            const double wv = (double)load1_ro(wp, o + e);
            swo = fma(wv, (double)x[e], swo);
            sww = fma(wv, wv, sww);
          }
        }
    }
  }
  if (wp != nullptr) block_partial3<kTileThreads>(osq, swo, sww, args.st, mt.onorm_slot, mt.hook_slot, job.part);
  else block_partial2<kTileThreads>(osq, 0.0, args.st, mt.onorm_slot, job.part);
}

namespace {
template <typename ST, typename OT, bool FOLD>
void launch_tile_f(int TP, dim3 grid, const TileMat* mats, const TileJob* jobs, const TileArgs& args, hipStream_t s) {
  if (TP == 64) hipLaunchKernelGGL((k_tile_ns<ST, OT, 64, FOLD>), grid, dim3(kTileThreads), 0, s, mats, jobs, args);
  else hipLaunchKernelGGL((k_tile_ns<ST, OT, 128, FOLD>), grid, dim3(kTileThreads), 0, s, mats, jobs, args);
}
template <typename ST, typename OT>
void launch_tile_t(int TP, dim3 grid, const TileMat* mats, const TileJob* jobs, const TileArgs& args, hipStream_t s) {
  // fp32 operands never fold (the master is the operand)
  if (sizeof(OT) == 2 && args.fold) launch_tile_f<ST, OT, sizeof(OT) == 2>(TP, grid, mats, jobs, args, s);
  else launch_tile_f<ST, OT, false>(TP, grid, mats, jobs, args, s);
}
}  // namespace

hipError_t launch_tile256_ns(const TileMat* mats, const TileJob* jobs, int njobs, const TileArgs& args,
                             hipStream_t s);

hipError_t launch_tile_ns(int state_dt, int op_dt, const TileMat* mats, const TileJob* jobs, int njobs,
                          const TileArgs& args, hipStream_t s) {
  if (njobs <= 0) return hipSuccess;
  if (args.T > kTileResidentMax) {  // 128 < T <= 256: the fused 256-tile kernel (bf16 state and operands)
    if (state_dt != DT_BF16 || op_dt != DT_BF16) return hipErrorInvalidValue;
    return launch_tile256_ns(mats, jobs, njobs, args, s);
  }
  if (args.T < 1 || args.K < 0 || args.K > kTileMaxK) return hipErrorInvalidValue;
  const int TP = args.T <= 64 ? 64 : 128;
  const dim3 grid(njobs);
  if (state_dt == DT_BF16 && op_dt == DT_BF16) launch_tile_t<bf16_t, bf16_t>(TP, grid, mats, jobs, args, s);
  else if (state_dt == DT_BF16) launch_tile_t<bf16_t, float>(TP, grid, mats, jobs, args, s);
  else if (op_dt == DT_BF16) launch_tile_t<float, bf16_t>(TP, grid, mats, jobs, args, s);
  else launch_tile_t<float, float>(TP, grid, mats, jobs, args, s);
  return hipGetLastError();
}

}  // namespace muonh
