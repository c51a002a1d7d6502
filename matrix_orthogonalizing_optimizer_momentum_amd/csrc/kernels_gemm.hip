// Grouped MFMA GEMM engine for the Newton-Schulz iteration (gfx950).
//
// One Newton-Schulz iteration (Muon explainer, Newton-Schulz section,
// Equation 6 and the code section) is three products on the small (r x r)
// Gram side of each r x s matrix X:
//   G1  A = X X^T                      (scaled by 1/(||M||+eps)^2 on the first
//                                       iteration, where X0 = M unscaled)
//   G2  B = b A + c A A                (A symmetric)
//   G3  X <- a X + B X                 (scaled by 1/(||M||+eps) on the first
//                                       iteration; the last iteration writes O
//                                       in the caller's layout and its sum of
//                                       squares)
// X lives only as X^T (s rows of r, both sides zero-padded to 64) in a 16-bit
// storage type (bf16 X0^T from the momentum pass; with fp16 iterates every
// later X^T, A and B in fp16) or fp32, plus an fp32 master copy in the same
// layout when requested.  A launch reads its operands in one type and stores
// its product in another (bf16 -> fp16 for the first update under fp16
// iterates).
// Every product is D[i][j] = sum_k P[i][k] Q[j][k]:
//   G2 reads A twice and G3 reads B and X^T with K-contiguous rows;
//   G1 reads X^T tiles [k][m] and forms K-contiguous MFMA fragments with
//   gfx950's transposing LDS read (ds_read_b64_tr_b16) for bf16, or plain
//   column reads for fp32.
// G3's accumulator is seeded with a X read from X^T (4 consecutive rows of X
// per lane are contiguous in X^T), and the new X^T (and fp32 master) is
// stored straight from the accumulator layout with packed 8 / 16-byte stores.
// A and B are symmetric: G1 and G2 compute tiles on or above the diagonal and
// mirror the rest.
//
// A launch covers every unit (matrix or HiMuon tile) of a chunk through a job
// list of BM x BN output tiles; job order is remapped so that the jobs one XCD
// runs are contiguous in the list (operand panels shared in its L2).
// Operands are bf16 (v_mfma_f32_32x32x16_bf16), fp16
// (v_mfma_f32_32x32x16_f16, the same rate) or fp32 (v_mfma_f32_32x32x2_f32),
// accumulation is fp32.  Two main loops:
//   - 128 x 128 tiles (4 waves, two workgroups per CU): LDS stages double
//     buffered behind a register prefetch ring of 16-byte global loads, MFMA
//     fragments double buffered in registers (the same loop on 64 x 64 tiles
//     for fp32 units of side <= 256, whose products are latency-bound);
//   - 256 x 256 tiles with bf16 operands (8 waves, one workgroup per CU): an
//     8-wave ping-pong, waves w and w + 4 alternating between reading a half
//     stage's fragments from LDS and running its MFMAs, with the operands
//     brought in by direct global -> LDS loads interleaved with the MFMAs.
// The epilogues (seeded accumulators, mirrored symmetric tiles, X^T stored
// from registers, O in the caller's layout) are shared.
#include <type_traits>

#include "common.h"

namespace muonh {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

template <typename T> struct Mf;
template <> struct Mf<bf16_t> {
  static constexpr int KSTEP = 16;   // K per MFMA
  static constexpr int VEC = 8;      // elements per 16-byte chunk
  static constexpr int PAD = 8;      // LDS row padding, elements (16 bytes)
  using frag = bf16x8_t;
  static __device__ __forceinline__ frag ld(const bf16_t* p) { return *reinterpret_cast<const bf16x8_t*>(p); }
  static __device__ __forceinline__ f32x16_t mma(frag a, frag b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mf<f16_t> {
  static constexpr int KSTEP = 16;
  static constexpr int VEC = 8;
  static constexpr int PAD = 8;
  using frag = f16x8_t;
  static __device__ __forceinline__ frag ld(const f16_t* p) { return *reinterpret_cast<const f16x8_t*>(p); }
  static __device__ __forceinline__ f32x16_t mma(frag a, frag b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mf<float> {
  static constexpr int KSTEP = 2;
  static constexpr int VEC = 4;
  static constexpr int PAD = 4;
  using frag = float;
  static __device__ __forceinline__ frag ld(const float* p) { return *p; }
  static __device__ __forceinline__ f32x16_t mma(frag a, frag b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

enum { kG1 = 0, kG2 = 1, kG3 = 2 };

struct NsIterArgs {
  float a, b, c;      // this iteration's coefficients
  float eps;          // pre-scale eps
  int first;          // iteration 0: fold the pre-scale
  int last;           // final iteration: write O and its norm
  int cur;            // X^T ping-pong index read this iteration (G3 writes the other)
  int no_mma;         // K == 0: O = X0 / (||X0|| + eps) through the G3 epilogue
  int master32;       // X32 mode: G3 keeps the fp32 master X^T in NsUnit::x32
  int seed32;         // the first G3 seeds a X0 from NsUnit::x32 (fp32 X0^T)
  int njobs;
  SlotTable st;
};

constexpr int kThreads = 256;


// s_waitcnt immediates (gfx9 field layout: vmcnt [3:0] and [15:14], expcnt
// [6:4], lgkmcnt [11:8]): wait on one counter, leave the others at maximum.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | (((N >> 4) & 3) << 14));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// 4 consecutive elements as float.
template <typename T16>
__device__ __forceinline__ void load4_16(const T16* p, int64_t i, float (&v)[4]) {
  const u32x2_t q = *reinterpret_cast<const MUONH_GLOBAL u32x2_t*>(gmem(p + i));
  v[0] = lo16<T16>(q[0]);
  v[1] = hi16<T16>(q[0]);
  v[2] = lo16<T16>(q[1]);
  v[3] = hi16<T16>(q[1]);
}
__device__ __forceinline__ void load4(const bf16_t* p, int64_t i, float (&v)[4]) { load4_16(p, i, v); }
__device__ __forceinline__ void load4(const f16_t* p, int64_t i, float (&v)[4]) { load4_16(p, i, v); }
__device__ __forceinline__ void load4(const float* p, int64_t i, float (&v)[4]) {
  const f32x4_t a = *reinterpret_cast<const MUONH_GLOBAL f32x4_t*>(gmem(p + i));
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
}
__device__ __forceinline__ void store4(bf16_t* p, int64_t i, const float (&v)[4]) {
  const u32x2_t w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  *reinterpret_cast<MUONH_GLOBAL u32x2_t*>(gmem(p + i)) = w;
}
__device__ __forceinline__ void store4(f16_t* p, int64_t i, const float (&v)[4]) {
  const u32x2_t w = {pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3])};
  *reinterpret_cast<MUONH_GLOBAL u32x2_t*>(gmem(p + i)) = w;
}
__device__ __forceinline__ void store4(float* p, int64_t i, const float (&v)[4]) {
  const f32x4_t a = {v[0], v[1], v[2], v[3]};
  *reinterpret_cast<MUONH_GLOBAL f32x4_t*>(gmem(p + i)) = a;
}

// Store n (<= N) output values of O (run-time dtype), vectorized when the
// caller's layout allows it; adds the squares of the stored (rounded)
// values to osq (fp64).
template <int N>
__device__ __forceinline__ void store_out(void* p, int64_t i, const float (&v)[N], int n, int dtype, bool vec,
                                          double& osq) {
  float rv[N];
  if (vec && n == N) {
#pragma unroll
    for (int e = 0; e < N; ++e) rv[e] = (dtype == DT_BF16) ? St<bf16_t>::round(v[e]) : v[e];
    if (N == 4) {
      if (dtype == DT_BF16) store4(reinterpret_cast<bf16_t*>(p), i, *reinterpret_cast<const float(*)[4]>(rv));
      else store4(reinterpret_cast<float*>(p), i, *reinterpret_cast<const float(*)[4]>(rv));
    } else {
      if (dtype == DT_BF16) store8(reinterpret_cast<bf16_t*>(p), i, *reinterpret_cast<const float(*)[8]>(rv));
      else store8(reinterpret_cast<float*>(p), i, *reinterpret_cast<const float(*)[8]>(rv));
    }
  } else {
#pragma unroll
    for (int e = 0; e < N; ++e) rv[e] = e < n ? store_dyn(p, i + e, v[e], dtype) : 0.f;
  }
#pragma unroll
  for (int e = 0; e < N; ++e) osq = fma((double)rv[e], (double)rv[e], osq);
}

// Two transposing LDS reads (gfx950 ds_read_b64_tr_b16) form one bf16 MFMA
// fragment: within each 16-lane group, lane j addresses row j / 4, elements
// 4 (j % 4) .. + 3 of a [k][m] tile, and lane i receives element i of rows
// 0..3 (4 consecutive k for one m); p1 covers the next 4 rows.
template <typename F>
__device__ __forceinline__ F ld_tr8(const uint16_t* p0, const uint16_t* p1) {
  typedef short i16x8_t __attribute__((ext_vector_type(8)));
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)p0);
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)p1);
  const i16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(F, v);
}

// Block tile BM x BN (BM == BN) on WGM x WGN waves, each wave (BM/WGM) x
// (BN/WGN) built from 32 x 32 MFMA tiles; BK elements of K per LDS stage.
// Register budgets keep two waves per SIMD: 128-tiles run two workgroups of
// 4 waves per CU, 256-tiles one workgroup of 8 waves.
template <typename T, typename TO, int PHASE, int BM, int BN, int BK, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) __attribute__((amdgpu_waves_per_eu(2))) void k_ns_gemm(
    const NsUnit* __restrict__ units, const GemmJob* __restrict__ jobs, NsIterArgs args) {
  using M = Mf<T>;
  static_assert(sizeof(T) == sizeof(TO), "the output storage has the operand's width");
  // 16-bit storage types of the operands and of the output (bf16 stand-ins
  // for fp32 instances, whose 16-bit paths are compiled out)
  using T16 = typename std::conditional<sizeof(T) == 2, T, bf16_t>::type;
  using TO16 = typename std::conditional<sizeof(TO) == 2, TO, bf16_t>::type;
  constexpr int NT = 64 * WGM * WGN;  // threads
  constexpr bool TR = PHASE == kG1;   // operands are X^T tiles stored [k][m]
  constexpr int VEC = M::VEC, KSTEP = M::KSTEP;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int MI = WM / 32, NI = WN / 32;
  // LDS operand tiles: K-contiguous rows [m][k] with pitch LDK, or (TR)
  // [k][m] rows of BM elements, row k rotated by ROT * (k % RN) elements so
  // that the rows one fragment read touches land in different banks.
  // 256-tiles with bf16 operands run the ping-pong main loop (below): no
  // row padding (direct loads write whole 1 KB runs), XOR-swizzled chunks.
  constexpr bool PP = sizeof(T) == 2 && WGM * WGN == 8;
  // G3 on the ping-pong loop keeps its operands in a ring of five 32 KB
  // slots instead of two 64 KB stages (see the main loop)
  constexpr bool RING5 = PP && PHASE == kG3;
  constexpr int LDK = PP ? BK : BK + M::PAD;
  constexpr int RN = sizeof(T) == 2 ? 4 : 2, ROT = 32;
  constexpr int PSZ = TR ? BK * BM : BM * LDK;  // elements per operand stage
  constexpr int QSZ = TR ? BK * BN : BN * LDK;
  constexpr int CPR = TR ? BM / VEC : BK / VEC;  // 16-byte chunks per LDS row
  constexpr int P_LOADS = BM * BK / VEC / NT;
  constexpr int Q_LOADS = BN * BK / VEC / NT;
  static_assert(BM == BN, "square block tiles");
  static_assert(BM * BK % (VEC * NT) == 0, "tile/thread mismatch");
  static_assert(BK % KSTEP == 0 && kPad % BK == 0, "K stage must divide the padding granule");
  static_assert(!TR || (BM % (ROT * RN) == 0 && BK % (RN * KSTEP / 2) == 0), "rotation layout");

  // Main loop: P and Q stages (double buffered).  The epilogue reuses the
  // same LDS for its fp32 slabs.
  constexpr int kStage = RING5 ? 5 * PSZ * (int)sizeof(T) : 2 * (PSZ + QSZ) * (int)sizeof(T);
  // Slab rows: fit the stage buffers, and keep the batched row-pass reads of
  // a slab (SLAB * BN / NT values per thread) within 64 registers.
  constexpr int SLAB_LDS = (BM * BN * 4 <= kStage) ? BM : ((BM / 2) * BN * 4 <= kStage ? BM / 2 : BM / 4);
  constexpr int SLAB_REG = 64 * NT / BN;
  constexpr int SLAB = SLAB_LDS < SLAB_REG ? SLAB_LDS : SLAB_REG;
  constexpr int kSmem = kStage > SLAB * BN * 4 ? kStage : SLAB * BN * 4;
  __shared__ __attribute__((aligned(16))) char smem[kSmem];
  T* const sP = reinterpret_cast<T*>(smem);  // [2][PSZ]
  T* const sQ = sP + 2 * PSZ;                // [2][QSZ]

  // XCD-aware job order: hardware deals blocks round-robin over 8 XCDs; give
  // each XCD a contiguous run of the job list.
  int job_id;
  {
    const int nj = args.njobs, bid = blockIdx.x;
    const int q = nj / 8, rem = nj % 8, xcd = bid % 8, loc = bid / 8;
    job_id = xcd * q + min(xcd, rem) + loc;
  }
  const GemmJob job = jobs[job_id];
  const NsUnit u = units[job.unit];
  const T* const xt_in = reinterpret_cast<const T*>(args.cur ? u.xt[1] : u.xt[0]);

  // operands: G1 X^T (as [k][m] tiles); G2 A, A; G3 B, X^T (K-contiguous rows)
  const T* P;
  const T* Q;
  int64_t ldP, ldQ;
  int Prows, Qrows, K;
  if (PHASE == kG1) {
    P = xt_in; Q = xt_in; ldP = ldQ = u.ld_r; Prows = Qrows = u.ld_s; K = u.ld_s;
  } else if (PHASE == kG2) {
    P = reinterpret_cast<const T*>(u.a); Q = P; ldP = ldQ = u.ld_r; Prows = Qrows = u.r; K = u.ld_r;
  } else {
    P = reinterpret_cast<const T*>(u.b); Q = xt_in;
    ldP = u.ld_r; ldQ = u.ld_r; Prows = u.r; Qrows = u.ld_s; K = u.ld_r;
  }
  const int row0 = job.tm * BM, col0 = job.tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  // Pre-scale of the first iteration, read now so its latency is hidden.
  double sig = 1.0;
  if (args.first) sig = 1.0 / (sqrt(args.st.sums[2 * u.norm_slot]) + (double)args.eps);

  // Accumulator seed.  G3 starts from a X (the a X term of the update; 1 * X0
  // for K = 0) and G2 from (b / c) A, so B = c (A A + (b / c) A) (c = 0: B =
  // b A with no product); G1 starts from zero.  In the accumulator layout a
  // lane holds rows m..m+3 of one column n: X(m..m+3, n) is X^T(n, m..m+3),
  // and A(m..m+3, n) is A(n, m..m+3), so each group of 4 is one 8 / 16-byte
  // load, issued before the first operand stage.
  const float g2_seed = args.c != 0.f ? args.b / args.c : args.b;
  const float g2_mul = args.c != 0.f ? args.c : 1.f;
  const int lrow = 4 * (lane >> 5), lcol = lane & 31;  // accumulator-layout offsets
  f32x16_t acc[MI][NI];
  auto zero_acc = [&] {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  };
  const int nstage = (args.no_mma || (PHASE == kG2 && args.c == 0.f)) ? 0 : K / BK;
  // With bf16 seeds on 128-tiles the seed is "late": it is held in registers
  // of its own and added after the main loop, so it never delays the first
  // MFMA.  The seed block of X^T (or of A) is a sub-block of this tile's own
  // Q operand, so it is copied out of the LDS stage that holds it (seed_pull
  // below) instead of being read from HBM a second time; with no stages
  // (K = 0) it is loaded directly.  fp32 master seeds and 256-tiles (no spare
  // registers) load into the accumulators up front.
  constexpr bool kLateSeed = sizeof(T) == 2 && MI * NI <= 4;
  u32x2_t seedv[kLateSeed ? MI : 1][kLateSeed ? NI : 1][4];
  bool late = false;
  // 256-tiles (ping-pong loop) start from zero accumulators: with bf16
  // seeds each wave adds its seed block while the half stage of Q that holds
  // it is in LDS; fp32 master seeds, and seeds with no stages, are added
  // after the main loop.
  bool pp_late = false, pp_after = false;
  const T* const seed_src = PHASE == kG2 ? reinterpret_cast<const T*>(u.a) : xt_in;
  const int seed_nlim = PHASE == kG2 ? u.r : u.ld_s;  // rows of the seed source
  const float seed_coef = PHASE == kG2 ? g2_seed : (args.no_mma ? 1.f : args.a);
  auto seed_off = [&](int i, int j, int q, bool& ok) -> int64_t {
    const int m0 = row0 + wm * WM + i * 32 + 8 * q + lrow, n = col0 + wn * WN + j * 32 + lcol;
    ok = n < seed_nlim && m0 < u.ld_r;
    return ok ? (int64_t)n * u.ld_r + m0 : 0;  // clamped: always in bounds
  };
  if (PHASE == kG1) {
    zero_acc();
  } else if (PP) {
    zero_acc();
    const bool m32 = PHASE == kG3 && u.x32 != nullptr && (args.first ? args.seed32 : args.master32);
    pp_late = nstage > 0 && !m32;
    pp_after = !pp_late;
  } else {
    // fp32 seed: the master X^T (X32 mode), or the fp32 X0^T on the first iteration
    const bool m32 = PHASE == kG3 && u.x32 != nullptr && (args.first ? args.seed32 : args.master32);
    const T* src = seed_src;
    const float coef = seed_coef;
    late = kLateSeed && !m32;
    if (late) {
      if constexpr (kLateSeed) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              bool ok;
              if (nstage > 0) seedv[i][j][q] = u32x2_t{0u, 0u};  // filled from LDS in the main loop
              else seedv[i][j][q] = *reinterpret_cast<const MUONH_GLOBAL u32x2_t*>(gmem(src) + seed_off(i, j, q, ok));
            }
      }
      zero_acc();
    } else if (m32) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            bool ok;
            const f32x4_t x = *reinterpret_cast<const MUONH_GLOBAL f32x4_t*>(gmem(u.x32) + seed_off(i, j, q, ok));
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][4 * q + e] = x[e];
          }
    } else {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            bool ok;
            float x[4];
            load4(src, seed_off(i, j, q, ok), x);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][4 * q + e] = x[e];
          }
    }
    if (!late) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            bool ok;
            (void)seed_off(i, j, q, ok);
            const float mul = ok ? coef : 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][4 * q + e] *= mul;
          }
    }
  }

  // Global prefetch ring: stage ks+NPF's loads are issued when stage ks
  // starts, so each load has NPF-1 stages of MFMA work to arrive before its
  // LDS store; LDS itself is double buffered.  The ring is indexed only by
  // compile-time constants (fully unrolled), so it lives in registers.
#ifndef MUONH_NPF
#define MUONH_NPF 1
#endif
  constexpr int NPF = (MI * NI >= 8) ? 1 : (PHASE == kG1 ? 2 : MUONH_NPF);  // G1 has no seed registers
  constexpr int NL = P_LOADS + Q_LOADS;
  u32x4_t ring[NPF][NL];
  // Per-thread load coordinates: a 32-bit byte offset from the operand's
  // base (fixed for the whole K loop; operands are below 2 GiB), and the
  // uniform step between stages, so each load is one scalar-base + vector
  // offset access.
  const char* const Pb = reinterpret_cast<const char*>(P);
  const char* const Qb = reinterpret_cast<const char*>(Q);
  uint32_t goff[NL];
  const int64_t kstride = TR ? (int64_t)BK * u.ld_r * (int64_t)sizeof(T) : (int64_t)BK * (int64_t)sizeof(T);
#pragma unroll
  for (int l = 0; l < NL; ++l) {
    const bool isp = l < P_LOADS;
    const int ll = isp ? l : l - P_LOADS;
    const int c = (tid + ll * NT) % CPR, rr = (tid + ll * NT) / CPR;
    int64_t e;
    if (TR) {
      // row rr of the stage (k), 8 consecutive m; chunks past the padded
      // width are clamped to its last chunk (they feed only outputs >= ld_r)
      const int mc = min((isp ? row0 : col0) + c * VEC, u.ld_r - VEC);
      e = (int64_t)rr * ldP + mc;
    } else {
      // Rows past the operand's edge are clamped to its last row instead of
      // masked: the loads stay branch-free, and those rows only feed output
      // rows / columns the epilogue writes as zeros or not at all.
      const int gr = isp ? min(row0 + rr, Prows - 1) : min(col0 + rr, Qrows - 1);
      e = (int64_t)gr * (isp ? ldP : ldQ) + c * VEC;
    }
    goff[l] = (uint32_t)(e * (int64_t)sizeof(T));
  }
#define MUONH_GLOAD(slot, ks)                                                                       \
  do {                                                                                              \
    const int64_t kofs_ = (int64_t)(ks) * kstride;                                                  \
    const MUONH_GLOBAL char* pk_ = gmem(Pb + kofs_);                                                \
    const MUONH_GLOBAL char* qk_ = gmem(Qb + kofs_);                                                \
    _Pragma("unroll") for (int l = 0; l < NL; ++l) ring[slot][l] =                                  \
        *reinterpret_cast<const MUONH_GLOBAL u32x4_t*>((l < P_LOADS ? pk_ : qk_) + goff[l]);        \
  } while (0)
#define MUONH_LSTORE(buf, slot)                                                                        \
  do {                                                                                                 \
    _Pragma("unroll") for (int l = 0; l < NL; ++l) {                                                   \
      const bool isp_ = l < P_LOADS;                                                                   \
      const int ll_ = isp_ ? l : l - P_LOADS;                                                          \
      const int c_ = (tid + ll_ * NT) % CPR, r_ = (tid + ll_ * NT) / CPR;                  \
      const int o_ = TR ? r_ * BM + ((c_ * VEC + ROT * (r_ % RN)) & (BM - 1)) : r_ * LDK + c_ * VEC;   \
      T* dst_ = isp_ ? sP + (buf) * PSZ + o_ : sQ + (buf) * QSZ + o_;                                  \
      *reinterpret_cast<u32x4_t*>(dst_) = ring[slot][l];                                              \
    }                                                                                                  \
  } while (0)

  // Per-lane fragment offsets inside an operand stage.
  int pofs[MI], qofs[NI];
  if (TR) {
    if (sizeof(T) == 2) {
      // lane = 16 g + j: rows 8 (g / 2) + j / 4 (+ 4 for the second read),
      // elements 16 (g % 2) + 4 (j % 4) of the 32-wide block
      const int j16 = lane & 15, g = lane >> 4;
      const int krow = 8 * (g >> 1) + (j16 >> 2);
      const int msub = 16 * (g & 1) + 4 * (j16 & 3) + ROT * (j16 >> 2);  // krow % 4 == j16 / 4
#pragma unroll
      for (int i = 0; i < MI; ++i) pofs[i] = krow * BM + ((wm * WM + i * 32 + msub) & (BM - 1));
#pragma unroll
      for (int j = 0; j < NI; ++j) qofs[j] = krow * BM + ((wn * WN + j * 32 + msub) & (BM - 1));
    } else {
      // fp32: lane reads k = lane / 32, m = lane % 32 (row k rotated by k % 2)
      const int krow = lane >> 5, msub = (lane & 31) + ROT * krow;
#pragma unroll
      for (int i = 0; i < MI; ++i) pofs[i] = krow * BM + ((wm * WM + i * 32 + msub) & (BM - 1));
#pragma unroll
      for (int j = 0; j < NI; ++j) qofs[j] = krow * BM + ((wn * WN + j * 32 + msub) & (BM - 1));
    }
  } else {
#pragma unroll
    for (int i = 0; i < MI; ++i) pofs[i] = (wm * WM + i * 32 + lcol) * LDK + (lane >> 5) * (KSTEP / 2);
#pragma unroll
    for (int j = 0; j < NI; ++j) qofs[j] = (wn * WN + j * 32 + lcol) * LDK + (lane >> 5) * (KSTEP / 2);
  }
  // Fragment of k-step kk from an operand stage.
  auto frag = [&](const T* stage, int ofs, int kk) -> typename M::frag {
    if constexpr (!TR) {
      return M::ld(stage + ofs + kk * KSTEP);
    } else if constexpr (sizeof(T) == 2) {
      const uint16_t* p = reinterpret_cast<const uint16_t*>(stage) + ofs + kk * KSTEP * BM;
      return ld_tr8<typename M::frag>(p, p + 4 * BM);
    } else {
      return stage[ofs + kk * KSTEP * BM];
    }
  };

  // One stage of MFMAs from LDS buffer buf; mid() runs after the first
  // k-step's MFMAs are issued (the next stage's LDS stores and global loads
  // then overlap with this stage's matrix work).
  auto compute = [&](int buf, auto&& mid) {
    const T* sp = sP + buf * PSZ;
    const T* sq = sQ + buf * QSZ;
    // Fragments double-buffered in registers: step kk+1's LDS reads are in
    // flight while step kk's MFMAs run.
    typename M::frag fa[2][MI], fb[2][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i) fa[0][i] = frag(sp, pofs[i], 0);
#pragma unroll
    for (int j = 0; j < NI; ++j) fb[0][j] = frag(sq, qofs[j], 0);
#pragma unroll
    for (int kk = 0; kk < BK / KSTEP; ++kk) {
      const int c = kk & 1;
      if (kk + 1 < BK / KSTEP) {
#pragma unroll
        for (int i = 0; i < MI; ++i) fa[c ^ 1][i] = frag(sp, pofs[i], kk + 1);
#pragma unroll
        for (int j = 0; j < NI; ++j) fb[c ^ 1][j] = frag(sq, qofs[j], kk + 1);
      }
      // Fence: the next step's reads are issued before this step's MFMAs
      // (the default schedule sinks each read next to its use and waits).
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) acc[i][j] = M::mma(fa[c][i], fb[c][j], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
      if (kk == 0) {
        mid();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Seed rows of accumulator block i (rows row0 + wm*WM + i*32 .. +31, i.e.
  // K indices of this tile's Q operand) sit in one K stage; during that stage
  // each lane copies its 4-row groups out of the Q buffer: Q row n holds
  // X^T(n, m) (G3) or A(n, m) (G2).
  auto seed_pull = [&](int buf, int ks) {
    if constexpr (kLateSeed && PHASE != kG1) {
      if (!late) return;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int rb = row0 + wm * WM + i * 32;
        if (rb / BK != ks) continue;  // uniform per wave
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const T* p = sQ + buf * QSZ + (wn * WN + j * 32 + lcol) * LDK + (rb % BK) + 8 * q + lrow;
            seedv[i][j][q] = *reinterpret_cast<const u32x2_t*>(p);
          }
      }
    }
  };

  if constexpr (RING5) {
    if (nstage > 0) {
      // The ping-pong of the two-stage loop below (groups 0 and 1 one phase
      // apart, memory and compute phases of half a 64-deep stage, a barrier
      // of all 8 waves after every phase), with the operands in a ring of
      // five 32 KB slots, each the P or the Q of a stage: stage s uses slots
      // 2 s and 2 s + 1 (mod 5).  The slots of stage ks - 1 (last read in
      // phase 4 ks - 1) receive Q of stage ks + 1 (phases 4 ks, 4 ks + 1) and
      // P of stage ks + 2 (phases 4 ks + 2, 4 ks + 3); P of stage ks + 1 came
      // during stage ks - 1.  So every compute phase carries four 1 KB
      // direct loads per wave, one after every fourth MFMA, and at the end of
      // phase 4 ks + 3 each wave waits for all but its newest four loads
      // (everything of stage ks + 1).  Measured against the two-stage loop:
      // faster for G3, slower for the symmetric G1 / G2, hence G3 only.
      static_assert(BM == 256 && PSZ == QSZ && BK == 64, "ping-pong layout: square 256-tiles, 64-deep stages");
      constexpr int SLOT_B = PSZ * (int)sizeof(T);
      constexpr int NRUN = SLOT_B / 1024;  // 1 KB direct loads per operand slot
      constexpr int RPW = NRUN / 8;        // per wave and phase
      constexpr int CPRK = BK / VEC;       // 16-byte chunks per K-contiguous row
      constexpr int RPR = 64 / CPRK;       // K-contiguous rows per run
      static_assert(NRUN * 1024 == SLOT_B && RPW * 8 == NRUN && 5 * SLOT_B <= kSmem, "slot layout");
      static_assert(CPRK == 8 && RPW == 4, "swizzle: 8 chunks per row; four loads per wave and phase");
      constexpr int NKH = BK / KSTEP / 2;  // k-steps per half stage
      auto swz = [](int r) { return (r >> 1) & 7; };
      const int wv = __builtin_amdgcn_readfirstlane(wave);
      const int grp = wv >> 2;
      auto slot_p = [&](int ks) { return smem + ((2 * ks) % 5) * SLOT_B; };
      auto slot_q = [&](int ks) { return smem + ((2 * ks + 1) % 5) * SLOT_B; };
      // A wave's loads of one operand slot: runs 16 grp + (wave % 4) + 4 p,
      // p < 4, each from a per-lane byte offset (the wave's first run, stage
      // 0) plus the uniform p * rstride.  Operand buffers are padded to whole
      // 256-row tiles, so no run is clamped.
      uint32_t voff[2];
      int64_t rstride;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int ii = 16 * grp + (wv & 3);
        const int64_t ld = h == 0 ? ldP : ldQ;
        const int base = h == 0 ? row0 : col0;
        const int rr = RPR * ii + lane / CPRK, pc = lane % CPRK;
        const int c = pc ^ swz(rr);
        const int64_t e = (int64_t)(base + rr) * ld + c * VEC;
        rstride = 4 * RPR * ld * (int64_t)sizeof(T);
        voff[h] = (uint32_t)(e * (int64_t)sizeof(T));
      }
      const int run0 = 16 * grp + (wv & 3);
      // run run0 + 4 p of operand h (0: P, 1: Q) of stage ks
      auto dma_run = [&](int ks, int h, int p) {
        const char* src = (h == 0 ? Pb : Qb) + (int64_t)ks * kstride + p * rstride;
        char* const dst = (h == 0 ? slot_p(ks) : slot_q(ks)) + (run0 + 4 * p) * 1024;
        __builtin_amdgcn_global_load_lds((MUONH_GLOBAL void*)(gmem(src) + voff[h]),
                                         (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
      };
      int xk[2 * NKH];
#pragma unroll
      for (int kk = 0; kk < 2 * NKH; ++kk) xk[kk] = ((2 * kk + (lane >> 5)) ^ swz(lcol)) * VEC;
      int pb[MI], qb[NI];
#pragma unroll
      for (int i = 0; i < MI; ++i) pb[i] = (wm * WM + i * 32 + lcol) * BK;
#pragma unroll
      for (int j = 0; j < NI; ++j) qb[j] = (wn * WN + j * 32 + lcol) * BK;
      typename M::frag fa[NKH][MI], fb[NKH][NI];
      auto read_half = [&](int ks, int sh) {
        const T* sp = reinterpret_cast<const T*>(slot_p(ks));
        const T* sq = reinterpret_cast<const T*>(slot_q(ks));
#pragma unroll
        for (int h = 0; h < NKH; ++h) {
          const int kk = NKH * sh + h;
#pragma unroll
          for (int i = 0; i < MI; ++i) fa[h][i] = M::ld(sp + pb[i] + xk[kk]);
#pragma unroll
          for (int j = 0; j < NI; ++j) fb[h][j] = M::ld(sq + qb[j] + xk[kk]);
        }
      };
      // Seed rows of accumulator block i are the 32 K rows of the half stage
      // with 32 (2 ks + sh) == row0 + wm * WM + i * 32: Q row n holds
      // X^T(n, m), and a lane's 4 rows m are one 8-byte piece of it.
      auto seed_pull_ring = [&](int ks, int sh) {
        if (!pp_late) return;
        const T* sq = reinterpret_cast<const T*>(slot_q(ks));
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          if (ks * BK + 32 * sh != row0 + wm * WM + i * 32) continue;  // uniform per wave
#pragma unroll
          for (int j = 0; j < NI; ++j) {
            const int nl = wn * WN + j * 32 + lcol;
            const float mul = col0 + nl < seed_nlim ? seed_coef : 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const u32x2_t w = *reinterpret_cast<const u32x2_t*>(sq + nl * BK + ((4 * sh + q) ^ swz(nl)) * VEC + lrow);
              acc[i][j][4 * q + 0] = fmaf(mul, lo16<T16>(w[0]), acc[i][j][4 * q + 0]);
              acc[i][j][4 * q + 1] = fmaf(mul, hi16<T16>(w[0]), acc[i][j][4 * q + 1]);
              acc[i][j][4 * q + 2] = fmaf(mul, lo16<T16>(w[1]), acc[i][j][4 * q + 2]);
              acc[i][j][4 * q + 3] = fmaf(mul, hi16<T16>(w[1]), acc[i][j][4 * q + 3]);
            }
          }
        }
      };
      // the half stage's MFMAs with this wave's four loads of operand lh of
      // stage lks in between (none for lks < 0)
      constexpr int NMF = NKH * MI * NI, MPL = NMF / RPW;
      static_assert(MPL * RPW == NMF, "loads spread evenly over the MFMAs");
      auto mma_half = [&](int lks, int lh) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int t = 0; t < NMF; ++t) {
          const int h = t / (MI * NI), i = (t / NI) % MI, j = t % NI;
          acc[i][j] = M::mma(fa[h][i], fb[h][j], acc[i][j]);
          if (t % MPL == MPL - 1) {
            __builtin_amdgcn_sched_barrier(0);
            if (lks >= 0) dma_run(lks, lh, t / MPL);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
      };
      auto bar = [] {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
      };
      // before the loop: P and Q of stage 0 and P of stage 1; wait for stage 0
#pragma unroll
      for (int p = 0; p < RPW; ++p) {
        dma_run(0, 0, p);
        dma_run(0, 1, p);
      }
      if (nstage > 1) {
#pragma unroll
        for (int p = 0; p < RPW; ++p) dma_run(1, 0, p);
        wait_vmcnt<RPW>();
      } else {
        wait_vmcnt<0>();
      }
      bar();
      // end of phase 4 ks + 3: all of stage ks + 1 has landed (only this
      // wave's loads of P of stage ks + 2 may still be in flight)
      auto wait_next = [&](int ks) {
        if (ks + 2 < nstage) wait_vmcnt<RPW>();
        else wait_vmcnt<0>();
      };
      if (grp == 0) {
        for (int ks = 0; ks < nstage; ++ks) {
          read_half(ks, 0);                                // phase 4 ks
          seed_pull_ring(ks, 0);
          wait_lgkmcnt0();
          bar();
          mma_half(ks + 1 < nstage ? ks + 1 : -1, 1);      // phase 4 ks + 1
          bar();
          read_half(ks, 1);                                // phase 4 ks + 2
          seed_pull_ring(ks, 1);
          wait_lgkmcnt0();
          bar();
          mma_half(ks + 2 < nstage ? ks + 2 : -1, 0);      // phase 4 ks + 3
          wait_next(ks);
          bar();
        }
      } else {
        for (int ks = 0; ks < nstage; ++ks) {
          if (ks > 0) {
            mma_half(ks + 1 < nstage ? ks + 1 : -1, 1);    // phase 4 ks
          } else if (nstage > 1) {
#pragma unroll
            for (int p = 0; p < RPW; ++p) dma_run(1, 1, p);
          }
          bar();
          read_half(ks, 0);                                // phase 4 ks + 1
          seed_pull_ring(ks, 0);
          wait_lgkmcnt0();
          bar();
          mma_half(ks + 2 < nstage ? ks + 2 : -1, 0);      // phase 4 ks + 2
          bar();
          read_half(ks, 1);                                // phase 4 ks + 3
          seed_pull_ring(ks, 1);
          wait_lgkmcnt0();
          wait_next(ks);
          bar();
        }
        mma_half(-1, 0);
      }
    }
  } else if constexpr (PP) {
    if (nstage > 0) {
      // Ping-pong: waves w and w + 4 share a SIMD.  Group 0 (waves 0-3) and
      // group 1 (waves 4-7) alternate between a memory phase (fragments of
      // half a stage, LDS -> registers) and a compute phase (that half
      // stage's MFMAs from registers), one phase apart, so one wave of each
      // SIMD feeds the matrix core while the other moves data; every phase
      // ends at a barrier of all 8 waves.
      //
      // LDS holds two stages [P | Q] of BK = 64 (128-byte rows: direct loads
      // of whole 128-byte row segments run at close to twice the rate of
      // 64-byte ones).  Phases of stage ks are 4 ks + 0..3 (group 0: memory
      // half 0, compute, memory half 1, compute; group 1 one phase behind).
      // Stage ks + 1 overwrites the buffer of stage ks - 1, whose last reads
      // (group 1, half 1) ended at phase 4 ks - 1.  Its direct global -> LDS
      // loads (group 0: the P half, group 1: the Q half, eight 1 KB runs per
      // wave) ride in the compute phases 4 ks (group 1) and 4 ks + 1
      // (group 0), one after every other MFMA, so their issue (the texture
      // path takes about 16 cycles per run) overlaps matrix work; both
      // groups wait for theirs at the end of phase 4 ks + 3, before the
      // stage's first read at phase 4 ks + 4.
      //
      // A 1 KB direct load writes lane l's 16 bytes at byte 16 l of the run,
      // so the global source of each lane is permuted to realise the XOR
      // swizzle of K-contiguous rows or the rotation of the transposed tiles.
      static_assert(BM == 256 && PSZ == QSZ && BK == 64, "ping-pong layout: square 256-tiles, 64-deep stages");
      constexpr int STAGE_B = (PSZ + QSZ) * (int)sizeof(T);
      constexpr int NDMA = STAGE_B / 1024;  // 1 KB direct loads per stage
      constexpr int DPW = NDMA / 8;         // per wave: a quarter of its group's half
      constexpr int CPRK = BK / VEC;        // 16-byte chunks per K-contiguous row
      constexpr int RPR = 64 / CPRK;        // K-contiguous rows per run
      static_assert(NDMA * 1024 == STAGE_B && DPW * 8 == NDMA && 2 * STAGE_B <= kSmem, "stage layout");
      static_assert(CPRK == 8, "swizzle: 8 chunks per row");
      constexpr int NKH = BK / KSTEP / 2;   // k-steps per half stage
      // Swizzle of K-contiguous rows: chunk c of row r sits at c ^ swz(r),
      // which spreads any 16 consecutive rows of one chunk over all banks.
      auto swz = [](int r) { return (r >> 1) & 7; };
      const int wv = __builtin_amdgcn_readfirstlane(wave);
      const int grp = wv >> 2;
      // A wave's runs are (wave % 4) + 4 p of its group's operand; run
      // (wave % 4) + 4 p is read from a per-lane byte offset (p = 0, stage
      // 0) plus the uniform p * rstride (the swizzle and rotation terms
      // depend only on the run modulo 4).  Operand buffers are padded to
      // whole 256-row tiles (and the transposed tiles' column overrun), so
      // no run is clamped.
      uint32_t voff;
      int64_t rstride;
      {
        const int ii = wv & 3;
        const int64_t ld = grp == 0 ? ldP : ldQ;
        const int base = grp == 0 ? row0 : col0;
        int64_t e;
        if (TR) {
          // two rows k of 256 elements per run; physical chunk pc holds
          // logical chunk (pc - 4 (k % 4)) % 32
          const int k = 2 * ii + (lane >> 5), pc = lane & 31;
          const int c = (pc - 4 * (k & 3)) & 31;
          e = (int64_t)k * ld + base + c * VEC;
          rstride = 8 * ld * (int64_t)sizeof(T);
        } else {
          const int rr = RPR * ii + lane / CPRK, pc = lane % CPRK;
          const int c = pc ^ swz(rr);
          e = (int64_t)(base + rr) * ld + c * VEC;
          rstride = 4 * RPR * ld * (int64_t)sizeof(T);
        }
        voff = (uint32_t)(e * (int64_t)sizeof(T));
      }
      const char* const opb = grp == 0 ? Pb : Qb;
      const int half = (grp == 0 ? 0 : PSZ * (int)sizeof(T)) + (wv & 3) * 1024;
      // run (wave % 4) + 4 p of stage ks
      auto dma_run = [&](int ks, int p) {
        const char* src = opb + (int64_t)ks * kstride + p * rstride;
        __builtin_amdgcn_global_load_lds((MUONH_GLOBAL void*)(gmem(src) + voff),
                                         (__attribute__((address_space(3))) void*)(smem + (ks & 1) * STAGE_B + half +
                                                                                   4 * p * 1024),
                                         16, 0, 0);
      };
      auto dma = [&](int ks) {
#pragma unroll
        for (int p = 0; p < DPW; ++p) dma_run(ks, p);
      };
      // fragment offsets (elements) inside a stage's P / Q halves
      int xk[2 * NKH];
#pragma unroll
      for (int kk = 0; kk < 2 * NKH; ++kk) xk[kk] = ((2 * kk + (lane >> 5)) ^ swz(lcol)) * VEC;
      int pb[MI], qb[NI];
#pragma unroll
      for (int i = 0; i < MI; ++i) pb[i] = TR ? pofs[i] : (wm * WM + i * 32 + lcol) * BK;
#pragma unroll
      for (int j = 0; j < NI; ++j) qb[j] = TR ? qofs[j] : (wn * WN + j * 32 + lcol) * BK;
      typename M::frag fa[NKH][MI], fb[NKH][NI];
      // fragments of half sh (k-steps NKH sh ..) of stage ks
      auto read_half = [&](int ks, int sh) {
        const T* sp = reinterpret_cast<const T*>(smem + (ks & 1) * STAGE_B);
        const T* sq = sp + PSZ;
#pragma unroll
        for (int h = 0; h < NKH; ++h) {
          const int kk = NKH * sh + h;
#pragma unroll
          for (int i = 0; i < MI; ++i) fa[h][i] = TR ? frag(sp, pb[i], kk) : M::ld(sp + pb[i] + xk[kk]);
#pragma unroll
          for (int j = 0; j < NI; ++j) fb[h][j] = TR ? frag(sq, qb[j], kk) : M::ld(sq + qb[j] + xk[kk]);
        }
      };
      // Seed rows of accumulator block i are the 32 K rows of the half stage
      // with 32 (2 ks + sh) == row0 + wm * WM + i * 32: Q row n holds
      // X^T(n, m) (G3) or A(n, m) (G2), and a lane's 4 rows m are one 8-byte
      // piece of it.
      auto seed_pull_pp = [&](int ks, int sh) {
        if constexpr (PHASE != kG1) {
          if (!pp_late) return;
          const T* sq = reinterpret_cast<const T*>(smem + (ks & 1) * STAGE_B) + PSZ;
#pragma unroll
          for (int i = 0; i < MI; ++i) {
            if (ks * BK + 32 * sh != row0 + wm * WM + i * 32) continue;  // uniform per wave
#pragma unroll
            for (int j = 0; j < NI; ++j) {
              const int nl = wn * WN + j * 32 + lcol;
              // rows m of a stage are below K = ld_r; columns n past the
              // seed source's rows get no seed
              const float mul = col0 + nl < seed_nlim ? seed_coef : 0.f;
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const u32x2_t w =
                    *reinterpret_cast<const u32x2_t*>(sq + nl * BK + ((4 * sh + q) ^ swz(nl)) * VEC + lrow);
                acc[i][j][4 * q + 0] = fmaf(mul, lo16<T16>(w[0]), acc[i][j][4 * q + 0]);
                acc[i][j][4 * q + 1] = fmaf(mul, hi16<T16>(w[0]), acc[i][j][4 * q + 1]);
                acc[i][j][4 * q + 2] = fmaf(mul, lo16<T16>(w[1]), acc[i][j][4 * q + 2]);
                acc[i][j][4 * q + 3] = fmaf(mul, hi16<T16>(w[1]), acc[i][j][4 * q + 3]);
              }
            }
          }
        }
      };
      // The half stage's MFMAs; with lks >= 0 this wave's runs of stage lks
      // are issued in between, one after every MPL MFMAs.
      constexpr int NMF = NKH * MI * NI, MPL = NMF / DPW;
      static_assert(MPL * DPW == NMF, "loads spread evenly over the MFMAs");
      auto mma_half = [&](int lks) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int t = 0; t < NMF; ++t) {
          const int h = t / (MI * NI), i = (t / NI) % MI, j = t % NI;
          acc[i][j] = M::mma(fa[h][i], fb[h][j], acc[i][j]);
          if (t % MPL == MPL - 1) {
            __builtin_amdgcn_sched_barrier(0);
            if (lks >= 0) dma_run(lks, t / MPL);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
      };
      auto bar = [] {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
      };
      dma(0);
      wait_vmcnt<0>();
      bar();
      if (grp == 0) {
        for (int ks = 0; ks < nstage; ++ks) {
          read_half(ks, 0);                          // phase 4 ks
          seed_pull_pp(ks, 0);
          wait_lgkmcnt0();
          bar();
          mma_half(ks + 1 < nstage ? ks + 1 : -1);   // phase 4 ks + 1
          bar();
          read_half(ks, 1);                          // phase 4 ks + 2
          seed_pull_pp(ks, 1);
          wait_lgkmcnt0();
          bar();
          mma_half(-1);                              // phase 4 ks + 3
          wait_vmcnt<0>();
          bar();
        }
      } else {
        for (int ks = 0; ks < nstage; ++ks) {
          if (ks > 0) mma_half(ks + 1 < nstage ? ks + 1 : -1);  // phase 4 ks
          else if (nstage > 1) dma(1);
          bar();
          read_half(ks, 0);                          // phase 4 ks + 1
          seed_pull_pp(ks, 0);
          wait_lgkmcnt0();
          bar();
          mma_half(-1);                              // phase 4 ks + 2
          bar();
          read_half(ks, 1);                          // phase 4 ks + 3
          seed_pull_pp(ks, 1);
          wait_lgkmcnt0();
          wait_vmcnt<0>();
          bar();
        }
        mma_half(-1);
      }
    }
  } else if (nstage > 0) {
    // Stage s lives in ring slot s % NPF from its global load until its LDS
    // store.  While stage ks is computed from LDS buffer ks % 2, stage ks+1
    // is stored into the other buffer and its ring slot is refilled with
    // stage ks+1+NPF, so a load has NPF stages of work to arrive.  The loop
    // is straight-line (no conditionals, so the compiler's wait counts stay
    // exact): load indices are clamped to the last stage and a store past the
    // end only fills the unused buffer; the nstage % NPF tail is peeled.
#pragma unroll
    for (int p = 0; p < NPF; ++p) MUONH_GLOAD(p, min(p, nstage - 1));
    MUONH_LSTORE(0, 0);
    MUONH_GLOAD(0, min(NPF, nstage - 1));
    __syncthreads();
    const int ngroups = nstage / NPF;
    for (int g = 0; g < ngroups; ++g) {
#pragma unroll
      for (int j = 0; j < NPF; ++j) {
        const int ks = g * NPF + j;  // ks % NPF == j
        compute(ks & 1, [&] {
          seed_pull(ks & 1, ks);
          MUONH_LSTORE((ks + 1) & 1, (j + 1) % NPF);
          MUONH_GLOAD((j + 1) % NPF, min(ks + 1 + NPF, nstage - 1));
        });
        __syncthreads();
      }
    }
#pragma unroll
    for (int j = 0; j < NPF - 1; ++j) {
      const int ks = ngroups * NPF + j;
      if (ks < nstage) {
        compute(ks & 1, [&] {
          seed_pull(ks & 1, ks);
          if (ks + 1 < nstage) MUONH_LSTORE((ks + 1) & 1, (j + 1) % NPF);
        });
        __syncthreads();
      }
    }
  }
#undef MUONH_GLOAD
#undef MUONH_LSTORE

  if constexpr (PP && PHASE != kG1) {
    if (pp_after) {
      // fp32 master seeds (or no stages): from HBM, one accumulator row
      // block at a time
      const bool m32 = PHASE == kG3 && u.x32 != nullptr && (args.first ? args.seed32 : args.master32);
#pragma unroll
      for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            bool ok;
            const int64_t o = seed_off(i, j, q, ok);
            const float mul = ok ? seed_coef : 0.f;
            float x[4];
            if (m32) {
              const f32x4_t t = *reinterpret_cast<const MUONH_GLOBAL f32x4_t*>(gmem(u.x32) + o);
              x[0] = t[0]; x[1] = t[1]; x[2] = t[2]; x[3] = t[3];
            } else {
              load4(seed_src, o, x);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][4 * q + e] = fmaf(mul, x[e], acc[i][j][4 * q + e]);
          }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if constexpr (kLateSeed) {
    if (late) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            bool ok;
            (void)seed_off(i, j, q, ok);
            const float mul = ok ? seed_coef : 0.f;
            const u32x2_t w = seedv[i][j][q];
            acc[i][j][4 * q + 0] = fmaf(mul, lo16<T16>(w[0]), acc[i][j][4 * q + 0]);
            acc[i][j][4 * q + 1] = fmaf(mul, hi16<T16>(w[0]), acc[i][j][4 * q + 1]);
            acc[i][j][4 * q + 2] = fmaf(mul, lo16<T16>(w[1]), acc[i][j][4 * q + 2]);
            acc[i][j][4 * q + 3] = fmaf(mul, hi16<T16>(w[1]), acc[i][j][4 * q + 3]);
          }
    }
  }

  const int r = u.r;
  // ------------------------------------------------ G3, not the last iteration
  // The new X^T (and fp32 master) straight from the accumulators: rows
  // m..m+3 of column n are X^T(n, m..m+3).  Rows >= r and columns >= s are
  // zero padding.  For each pair of 8-row groups, v_permlane32_swap trades
  // the upper half-wave's first group for the lower half-wave's second, so
  // that every lane holds 8 consecutive rows (lanes l and l+32 then cover 16
  // adjacent rows of X^T row n) and stores them with one 16-byte access (two
  // for the fp32 master).  The swaps run with every lane active; only the
  // stores are guarded.
  if (PHASE == kG3 && !args.last) {
    TO* const xo = reinterpret_cast<TO*>(args.cur ? u.xt[0] : u.xt[1]);
    const int hi = lane >> 5;
    // Most waves' blocks lie inside the matrix, and all iterations but the
    // first have no pre-scale: that case runs a copy of the store loop with
    // neither the bounds tests nor the fp64 scaling (which the compiler
    // would otherwise evaluate for every value and select away).
    const bool inside = row0 + wm * WM + WM <= r && col0 + wn * WN + WN <= u.s;
    auto store_x = [&](auto fast_c) {
      constexpr bool fast = decltype(fast_c)::value;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          const int n = col0 + wn * WN + j * 32 + lcol;
#pragma unroll
          for (int pq = 0; pq < 2; ++pq) {
            float v[2][4];  // groups q = 2pq, 2pq+1 of this lane's rows
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int q = 2 * pq + h, m0 = row0 + wm * WM + i * 32 + 8 * q + lrow;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                float t = acc[i][j][4 * q + e];
                if constexpr (fast) {
                  v[h][e] = t;
                } else {
                  if (args.first) t = (float)((double)t * sig);
                  v[h][e] = (m0 + e < r && n < u.s) ? t : 0.f;
                }
              }
            }
            // after the swaps: rows row0 + wm*WM + i*32 + 16*pq + 8*hi + 0..7
            const int ms = row0 + wm * WM + i * 32 + 16 * pq + 8 * hi;
            const bool ok = fast || (n < u.ld_s && ms < u.ld_r);
            const int64_t o = (int64_t)(ok ? n : 0) * u.ld_r + (ok ? ms : 0);
            if constexpr (sizeof(T) == 2) {
              uint32_t w0 = pack16x2<TO16>(v[0][0], v[0][1]), w1 = pack16x2<TO16>(v[0][2], v[0][3]);
              uint32_t w2 = pack16x2<TO16>(v[1][0], v[1][1]), w3 = pack16x2<TO16>(v[1][2], v[1][3]);
              const auto s0 = __builtin_amdgcn_permlane32_swap(w0, w2, false, false);
              const auto s1 = __builtin_amdgcn_permlane32_swap(w1, w3, false, false);
              const u32x4_t pk = {s0[0], s1[0], s0[1], s1[1]};
              if (ok) *reinterpret_cast<MUONH_GLOBAL u32x4_t*>(gmem(reinterpret_cast<uint16_t*>(xo) + o)) = pk;
            } else {
              float vs[8];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[0][e]), __float_as_uint(v[1][e]),
                                                                 false, false);
                vs[e] = __uint_as_float(sw[0]);
                vs[4 + e] = __uint_as_float(sw[1]);
              }
              if (ok) store8(reinterpret_cast<float*>(xo), o, vs);
            }
            if (args.master32 && u.x32 != nullptr) {
              float vs[8];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[0][e]), __float_as_uint(v[1][e]),
                                                                 false, false);
                vs[e] = __uint_as_float(sw[0]);
                vs[4 + e] = __uint_as_float(sw[1]);
              }
              if (ok) store8(u.x32, o, vs);
            }
          }
        }
    };
    if (inside && !args.first) store_x(std::true_type{});
    else store_x(std::false_type{});
    return;
  }

  // ----------------------------------------------------------------- epilogue
  // G1 / G2 (A or B and their mirrored tiles) and the last G3 (O in the
  // caller's layout).  The fp32 tile goes through LDS in slabs of SLAB rows,
  // stored with its 16-byte granules XOR-swizzled by (row / 8) so that the
  // accumulator writes, the row reads (one granule per lane) and the column
  // reads (8 rows per lane) avoid bank conflicts.  Outputs are then written
  // with row-contiguous accesses: a row pass (A, B, O in X orientation) and a
  // column pass (mirrored A / B tiles, O when the caller's layout is X^T).
  float* Ct = reinterpret_cast<float*>(smem);
  constexpr int GPR = BN / 4;  // granules per tile row
  static_assert(GPR >= 16, "swizzle needs 16 granules per row");
  auto cidx = [](int rl, int cl) -> int { return rl * BN + ((((cl >> 2) ^ ((rl >> 3) & 15))) << 2) + (cl & 3); };

  double osq = 0.0;
  const bool mirror = (PHASE != kG3) && (job.tm != job.tn);  // symmetric outputs: also write the transpose
  const bool col_pass = (PHASE == kG3) ? (u.o_trans != 0) : mirror;
  constexpr int ROWS_PER_IT = NT / GPR;    // row pass: one granule (4 values) per thread
  constexpr int RB = SLAB / ROWS_PER_IT;         // row-pass iterations per slab
  constexpr int CPC = SLAB / 8;                  // column pass: 8-row chunks per slab column
  constexpr int COLS_PER_IT = NT / CPC;
  static_assert(SLAB % ROWS_PER_IT == 0 && NT % CPC == 0 && BN % COLS_PER_IT == 0, "epilogue shape");
  const int gran = tid % GPR, rsub = tid / GPR;
  const int q = tid % CPC, csub = tid / CPC;
  const bool o_vec = (u.o_dtype == DT_BF16) ? ((u.o_ld % 8) == 0 && ((uintptr_t)u.o_ptr % 16) == 0)
                                            : ((u.o_ld % 4) == 0 && ((uintptr_t)u.o_ptr % 16) == 0);
  TO* const out12 = reinterpret_cast<TO*>(PHASE == kG1 ? u.a : u.b);

  constexpr int NCOL_IT = BN / COLS_PER_IT;
#pragma unroll 1
  for (int sl = 0; sl < BM / SLAB; ++sl) {
    __syncthreads();  // LDS free (main loop or previous slab done)
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int rbase = wm * WM + i * 32;
      if (rbase / SLAB != sl) continue;  // uniform per wave
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int rl = rbase - sl * SLAB + 8 * (v >> 2) + lrow + (v & 3);
          const int cl = wn * WN + j * 32 + lcol;
          Ct[cidx(rl, cl)] = acc[i][j][v];
        }
    }
    __syncthreads();

    // ---- row pass
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const int rl = b * ROWS_PER_IT + rsub;
      const int grow = row0 + sl * SLAB + rl;
      const int cl = gran * 4;
      const int gcol = col0 + cl;
      float* cp = &Ct[cidx(rl, cl)];
      float v[4];
      {
        const float4 t = *reinterpret_cast<const float4*>(cp);
        v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
      }
      if (PHASE == kG1 || PHASE == kG2) {
        if (grow < r && gcol < u.ld_r) {
          if (PHASE == kG1) {
            const float sc = (float)(sig * sig);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (gcol + e < r) ? v[e] * sc : 0.f;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (gcol + e < r) ? g2_mul * v[e] : 0.f;
          }
          store4(out12, (int64_t)grow * u.ld_r + gcol, v);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = 0.f;
        }
      } else {
        // last G3: O = acc = a X + B X (times sig when it is also the first)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float t = v[e];
          if (args.first) t = (float)((double)t * sig);
          v[e] = t;
        }
        if (!u.o_trans && grow < u.o_rows) {
          const int nv = min(4, u.o_cols - gcol);
          if (nv > 0) store_out<4>(u.o_ptr, (int64_t)grow * u.o_ld + gcol, v, nv, u.o_dtype, o_vec, osq);
        }
      }
      if (col_pass) *reinterpret_cast<float4*>(cp) = make_float4(v[0], v[1], v[2], v[3]);
    }

    // ---- column pass: tile column cl, 8 slab rows per chunk
    if (col_pass) {
      __syncthreads();
#pragma unroll
      for (int it = 0; it < NCOL_IT; ++it) {
        const int cl = it * COLS_PER_IT + csub;
        const int gn = col0 + cl;
        const int gi = row0 + sl * SLAB + q * 8;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = Ct[cidx(q * 8 + e, cl)];
        if (PHASE == kG1 || PHASE == kG2) {
          // mirrored tile: row gn of A (or B), columns gi..gi+7
          if (gn < r && gi < u.ld_r) store8(out12, (int64_t)gn * u.ld_r + gi, v);
        } else if (gn < u.o_cols && gi < u.o_rows) {
          store_out<8>(u.o_ptr, (int64_t)gn * u.o_ld + gi, v, min(8, u.o_rows - gi), u.o_dtype, o_vec, osq);
        }
      }
    }
  }
  if (PHASE == kG3) {
    const int part = u.onorm_part0 + job.tm * u.g3_cols + job.tn;
    if constexpr (RING5) {
      // the static LDS of block_partial2 does not fit beside the slot ring:
      // use bytes past the epilogue's slabs
      static_assert(SLAB * BN * 4 + 2 * (NT / 64) * 8 <= kSmem, "reduction scratch");
      block_partial2_at<NT>(osq, 0.0, args.st, u.onorm_slot, part,
                            reinterpret_cast<double(*)[NT / 64]>(smem + SLAB * BN * 4));
    } else {
      block_partial2<NT>(osq, 0.0, args.st, u.onorm_slot, part);
    }
  }
}

// ---------------------------------------------------------------------------
// host launcher
// ---------------------------------------------------------------------------
// Tile configurations (planner.h): 0 = 128 x 128 on 2 x 2 waves, K stages of
// 64 (bf16 / fp16) or 32 (fp32); 1 = 256 x 256 on 4 x 2 waves (16-bit
// operands, large units); 2 = 64 x 64 on 2 x 2 waves (fp32 units of side
// <= 256).  op_dt is the operands' storage, out_dt that of the product this
// launch stores (A, B or the new X^T; the last update writes O in the
// caller's dtype whatever out_dt says): (bf16, bf16), (bf16, fp16),
// (fp16, fp16) and (fp32, fp32).
hipError_t launch_ns_gemm(int op_dt, int out_dt, int phase, int cfg, const NsUnit* units, const GemmJob* jobs,
                          int njobs, float a, float b, float c, float eps, int first, int last, int cur,
                          int no_mma, int master32, int seed32, const SlotTable& st, hipStream_t s) {
  if (njobs <= 0) return hipSuccess;
  NsIterArgs args{a, b, c, eps, first, last, cur, no_mma, master32, seed32, njobs, st};
  dim3 grid(njobs);
#define MUONH_LAUNCH(T, TO, PH, B, K, GM, GN) \
  hipLaunchKernelGGL((k_ns_gemm<T, TO, PH, B, B, K, GM, GN>), grid, dim3(64 * GM * GN), 0, s, units, jobs, args)
#define MUONH_PHASES(T, TO, B, K, GM, GN)                          \
  do {                                                             \
    if (phase == kG1) MUONH_LAUNCH(T, TO, kG1, B, K, GM, GN);      \
    else if (phase == kG2) MUONH_LAUNCH(T, TO, kG2, B, K, GM, GN); \
    else MUONH_LAUNCH(T, TO, kG3, B, K, GM, GN);                   \
  } while (0)
#define MUONH_CFGS16(T, TO)                                 \
  do {                                                      \
    if (cfg == 1) MUONH_PHASES(T, TO, 256, 64, 4, 2);       \
    else MUONH_PHASES(T, TO, 128, 64, 2, 2);                \
  } while (0)
  if (op_dt == DT_BF16 && out_dt == DT_BF16) {
    MUONH_CFGS16(bf16_t, bf16_t);
  } else if (op_dt == DT_BF16 && out_dt == DT_F16) {
    MUONH_CFGS16(bf16_t, f16_t);
  } else if (op_dt == DT_F16 && out_dt == DT_F16) {
    MUONH_CFGS16(f16_t, f16_t);
  } else if (op_dt == DT_F32 && out_dt == DT_F32) {
    if (cfg == 2) MUONH_PHASES(float, float, 64, 32, 2, 2);
    else MUONH_PHASES(float, float, 128, 32, 2, 2);
  } else {
    return hipErrorInvalidValue;
  }
#undef MUONH_CFGS16
#undef MUONH_PHASES
#undef MUONH_LAUNCH
  return hipGetLastError();
}

}  // namespace muonh
