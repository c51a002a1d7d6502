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
// Every product here is D[i][j] = sum_k P[i][k] Q[j][k] with both operands
// stored K-contiguous: G1 reads X twice, G2 reads A twice (A = A^T), G3 reads
// B and X^T.  X^T is kept as a second copy that G3's epilogue writes, so no
// operand is ever transposed on load.  A and B are symmetric, so G1 and G2
// only compute tiles on or above the diagonal and mirror the rest.
//
// A launch covers every unit (matrix or HiMuon tile) of a chunk through a job
// list of BM x BN output tiles; job order is remapped so that the jobs one XCD
// runs are contiguous in the list (operand panels shared in its L2).
// Operands are bf16 (v_mfma_f32_32x32x16_bf16) or fp32
// (v_mfma_f32_32x32x2_f32), accumulation is fp32, LDS stages are double
// buffered with a register prefetch of the next stage, and MFMA fragments are
// double buffered in registers.
#include "common.h"

namespace muonh {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
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
  int cur;            // X^T ping-pong index read by G3
  int no_mma;         // K == 0: O = X0 / (||X0|| + eps) through the G3 epilogue
  int njobs;
  SlotTable st;
};

constexpr int kThreads = 256;

// 4 consecutive elements as float.
__device__ __forceinline__ void load4(const bf16_t* p, int64_t i, float (&v)[4]) {
  const u32x2_t q = *reinterpret_cast<const MUONH_GLOBAL u32x2_t*>(gmem(p + i));
  v[0] = __uint_as_float(q[0] << 16);
  v[1] = __uint_as_float(q[0] & 0xffff0000u);
  v[2] = __uint_as_float(q[1] << 16);
  v[3] = __uint_as_float(q[1] & 0xffff0000u);
}
__device__ __forceinline__ void load4(const float* p, int64_t i, float (&v)[4]) {
  const f32x4_t a = *reinterpret_cast<const MUONH_GLOBAL f32x4_t*>(gmem(p + i));
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
}
__device__ __forceinline__ void store4(bf16_t* p, int64_t i, const float (&v)[4]) {
  const u32x2_t w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  *reinterpret_cast<MUONH_GLOBAL u32x2_t*>(gmem(p + i)) = w;
}
__device__ __forceinline__ void store4(float* p, int64_t i, const float (&v)[4]) {
  const f32x4_t a = {v[0], v[1], v[2], v[3]};
  *reinterpret_cast<MUONH_GLOBAL f32x4_t*>(gmem(p + i)) = a;
}

// Store n (<= 4 or 8) output values of O (run-time dtype), vectorized when
// the caller's layout allows it; returns the sum of squares of the stored
// (rounded) values.
__device__ __forceinline__ float store_out4(void* p, int64_t i, const float (&v)[4], int n, int dtype, bool vec) {
  float sq = 0.f;
  if (vec && n == 4) {
    float rv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) rv[e] = (dtype == DT_BF16) ? St<bf16_t>::round(v[e]) : v[e];
    if (dtype == DT_BF16) store4(reinterpret_cast<bf16_t*>(p), i, rv);
    else store4(reinterpret_cast<float*>(p), i, rv);
#pragma unroll
    for (int e = 0; e < 4; ++e) sq = fmaf(rv[e], rv[e], sq);
  } else {
    for (int e = 0; e < n; ++e) {
      const float sv = store_dyn(p, i + e, v[e], dtype);
      sq = fmaf(sv, sv, sq);
    }
  }
  return sq;
}
__device__ __forceinline__ float store_out8(void* p, int64_t i, const float (&v)[8], int n, int dtype, bool vec) {
  float sq = 0.f;
  if (vec && n == 8) {
    float rv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) rv[e] = (dtype == DT_BF16) ? St<bf16_t>::round(v[e]) : v[e];
    if (dtype == DT_BF16) store8(reinterpret_cast<bf16_t*>(p), i, rv);
    else store8(reinterpret_cast<float*>(p), i, rv);
#pragma unroll
    for (int e = 0; e < 8; ++e) sq = fmaf(rv[e], rv[e], sq);
  } else {
    for (int e = 0; e < n; ++e) {
      const float sv = store_dyn(p, i + e, v[e], dtype);
      sq = fmaf(sv, sv, sq);
    }
  }
  return sq;
}

// Block tile BM x BN, 4 waves in 2 x 2, each wave (BM/2) x (BN/2) built from
// 32 x 32 MFMA tiles; BK elements of K per LDS stage.
template <typename T, int PHASE, int BM, int BN, int BK>
__global__ __launch_bounds__(kThreads) void k_ns_gemm(const NsUnit* __restrict__ units,
                                                     const GemmJob* __restrict__ jobs, NsIterArgs args) {
  using M = Mf<T>;
  constexpr int VEC = M::VEC, KSTEP = M::KSTEP, LDK = BK + M::PAD;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int MI = WM / 32, NI = WN / 32;
  constexpr int CPR = BK / VEC;                          // 16-byte chunks per row
  constexpr int P_LOADS = BM * CPR / kThreads;           // per thread per stage
  constexpr int Q_LOADS = BN * CPR / kThreads;
  static_assert(BM * CPR % kThreads == 0 && BN * CPR % kThreads == 0, "tile/thread mismatch");
  static_assert(BK % KSTEP == 0 && kPad % BK == 0, "K stage must divide the padding granule");

  // Main loop: P and Q stages (double buffered).  The epilogue reuses the
  // same LDS for its fp32 slabs.
  constexpr int kStage = 2 * (BM + BN) * LDK * (int)sizeof(T);
  // Slab rows: fit the stage buffers, and keep the batched row-pass reads of
  // a slab (SLAB * BN / kThreads values per thread) within 64 registers.
  constexpr int SLAB_LDS = (BM * BN * 4 <= kStage) ? BM : ((BM / 2) * BN * 4 <= kStage ? BM / 2 : BM / 4);
  constexpr int SLAB_REG = 64 * kThreads / BN;
  constexpr int SLAB = SLAB_LDS < SLAB_REG ? SLAB_LDS : SLAB_REG;
  constexpr int kSmem = kStage > SLAB * BN * 4 ? kStage : SLAB * BN * 4;
  __shared__ __attribute__((aligned(16))) char smem[kSmem];
  T (*sP)[BM * LDK] = reinterpret_cast<T (*)[BM * LDK]>(smem);
  T (*sQ)[BN * LDK] = reinterpret_cast<T (*)[BN * LDK]>(smem + 2 * BM * LDK * sizeof(T));

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

  const T* P;
  const T* Q;
  int64_t ldP, ldQ;
  int Prows, Qrows, K;
  if (PHASE == kG1) {
    P = reinterpret_cast<const T*>(u.x); Q = P; ldP = ldQ = u.ld_s; Prows = Qrows = u.r; K = u.ld_s;
  } else if (PHASE == kG2) {
    P = reinterpret_cast<const T*>(u.a); Q = P; ldP = ldQ = u.ld_r; Prows = Qrows = u.r; K = u.ld_r;
  } else {
    P = reinterpret_cast<const T*>(u.b); Q = reinterpret_cast<const T*>((args.cur ? u.xt[1] : u.xt[0]));
    ldP = u.ld_r; ldQ = u.ld_r; Prows = u.r; Qrows = u.s; K = u.ld_r;
  }
  const int row0 = job.tm * BM, col0 = job.tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // Accumulator seed.  G3 starts from a X (the a X term of the update; 1 * X0
  // for K = 0) and G2 from (b / c) A, so B = c (A A + (b / c) A) (c = 0: B =
  // b A with no product); G1 starts from zero.  The seed is read in the
  // accumulator layout (32 lanes cover 32 consecutive columns) before the
  // first operand stage, so its latency hides behind the operand loads and
  // the epilogue issues no global reads.
  const float g2_seed = args.c != 0.f ? args.b / args.c : args.b;
  const float g2_mul = args.c != 0.f ? args.c : 1.f;
  f32x16_t acc[MI][NI];
  {
    const int rbase = row0 + wm * WM + 4 * (lane >> 5), cbase = col0 + wn * WN + (lane & 31);
    if (PHASE == kG1) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    } else if (PHASE == kG3 && !args.first && u.x32 != nullptr) {
      const MUONH_GLOBAL float* src = gmem(u.x32);
      const float coef = args.no_mma ? 1.f : args.a;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int row = rbase + i * 32 + 8 * (v >> 2) + (v & 3), col = cbase + j * 32;
            const bool ok = row < u.r && col < u.ld_s;
            const float x = src[ok ? (int64_t)row * u.ld_s + col : 0];  // clamped: always in bounds
            acc[i][j][v] = ok ? coef * x : 0.f;
          }
    } else {
      // G2: A (r x ld_r); G3: X in operand precision (first iteration, or no
      // fp32 master)
      const T* src = reinterpret_cast<const T*>(PHASE == kG2 ? u.a : u.x);
      const int64_t ld = PHASE == kG2 ? u.ld_r : u.ld_s;
      const float coef = PHASE == kG2 ? g2_seed : (args.no_mma ? 1.f : args.a);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int row = rbase + i * 32 + 8 * (v >> 2) + (v & 3), col = cbase + j * 32;
            const bool ok = row < u.r && col < ld;
            const float x = St<T>::ld(src, ok ? (int64_t)row * ld + col : 0);
            acc[i][j][v] = ok ? coef * x : 0.f;
          }
    }
  }

  const int nstage = (args.no_mma || (PHASE == kG2 && args.c == 0.f)) ? 0 : K / BK;
  // Global prefetch ring: stage ks+NPF's loads are issued when stage ks
  // starts, so each load has NPF-1 stages of MFMA work to arrive before its
  // LDS store; LDS itself is double buffered.  The ring is indexed only by
  // compile-time constants (fully unrolled), so it lives in registers.
#ifndef MUONH_NPF
#define MUONH_NPF 2
#endif
  constexpr int NPF = (MI * NI >= 16) ? 1 : MUONH_NPF;
  constexpr int NL = P_LOADS + Q_LOADS;
  u32x4_t ring[NPF][NL];
  // Per-thread load coordinates (fixed for the whole K loop).
  const MUONH_GLOBAL u32x4_t* gsrc[NL];
#pragma unroll
  for (int l = 0; l < NL; ++l) {
    const bool isp = l < P_LOADS;
    const int ll = isp ? l : l - P_LOADS;
    const int c = (tid + ll * kThreads) % CPR, rr = (tid + ll * kThreads) / CPR;
    // Rows past the operand's edge are clamped to its last row instead of
    // masked: the loads stay branch-free, and those rows only feed output
    // rows / columns >= r (or >= s) that the epilogue writes as zeros.
    const int gr = isp ? min(row0 + rr, Prows - 1) : min(col0 + rr, Qrows - 1);
    const T* base = isp ? P + (int64_t)gr * ldP : Q + (int64_t)gr * ldQ;
    gsrc[l] = reinterpret_cast<const MUONH_GLOBAL u32x4_t*>(gmem(base + c * VEC));
  }
#define MUONH_GLOAD(slot, ks)                                                 \
  do {                                                                        \
    const int kofs_ = (ks) * BK / VEC;                                        \
    _Pragma("unroll") for (int l = 0; l < NL; ++l) ring[slot][l] = gsrc[l][kofs_]; \
  } while (0)
#define MUONH_LSTORE(buf, slot)                                                              \
  do {                                                                                       \
    _Pragma("unroll") for (int l = 0; l < NL; ++l) {                                         \
      const bool isp_ = l < P_LOADS;                                                         \
      const int ll_ = isp_ ? l : l - P_LOADS;                                                \
      const int c_ = (tid + ll_ * kThreads) % CPR, r_ = (tid + ll_ * kThreads) / CPR;        \
      T* dst_ = isp_ ? &sP[buf][r_ * LDK + c_ * VEC] : &sQ[buf][r_ * LDK + c_ * VEC];        \
      *reinterpret_cast<u32x4_t*>(dst_) = ring[slot][l];                                    \
    }                                                                                        \
  } while (0)

  auto compute = [&](int buf) {
    const T* sp = sP[buf] + (wm * WM + (lane & 31)) * LDK + (lane >> 5) * (KSTEP / 2);
    const T* sq = sQ[buf] + (wn * WN + (lane & 31)) * LDK + (lane >> 5) * (KSTEP / 2);
    // Fragments double-buffered in registers: step kk+1's LDS reads are in
    // flight while step kk's MFMAs run.
    typename M::frag fa[2][MI], fb[2][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i) fa[0][i] = M::ld(sp + i * 32 * LDK);
#pragma unroll
    for (int j = 0; j < NI; ++j) fb[0][j] = M::ld(sq + j * 32 * LDK);
#pragma unroll
    for (int kk = 0; kk < BK / KSTEP; ++kk) {
      const int c = kk & 1;
      if (kk + 1 < BK / KSTEP) {
#pragma unroll
        for (int i = 0; i < MI; ++i) fa[c ^ 1][i] = M::ld(sp + i * 32 * LDK + (kk + 1) * KSTEP);
#pragma unroll
        for (int j = 0; j < NI; ++j) fb[c ^ 1][j] = M::ld(sq + j * 32 * LDK + (kk + 1) * KSTEP);
      }
      // Fence: the next step's reads are issued before this step's MFMAs
      // (the default schedule sinks each read next to its use and waits).
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) acc[i][j] = M::mma(fa[c][i], fb[c][j], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (nstage > 0) {
    // Straight-line steady state (no conditionals, so the compiler's wait
    // counts stay exact): the prefetch index is clamped to the last stage, a
    // clamped reload is never used; the nstage % NPF tail is peeled.
#pragma unroll
    for (int p = 0; p < NPF; ++p) MUONH_GLOAD(p, min(p, nstage - 1));
    MUONH_LSTORE(0, 0);
    __syncthreads();
    const int ngroups = nstage / NPF;
    for (int g = 0; g < ngroups; ++g) {
#pragma unroll
      for (int j = 0; j < NPF; ++j) {
        const int ks = g * NPF + j;  // ks % NPF == j
        MUONH_GLOAD(j, min(ks + NPF, nstage - 1));
        compute(ks & 1);
        MUONH_LSTORE((ks + 1) & 1, (j + 1) % NPF);  // after the last stage: an unused buffer
        __syncthreads();
      }
    }
#pragma unroll
    for (int j = 0; j < NPF - 1; ++j) {
      const int ks = ngroups * NPF + j;
      if (ks < nstage) {
        compute(ks & 1);
        if (ks + 1 < nstage) {
          MUONH_LSTORE((ks + 1) & 1, (j + 1) % NPF);
          __syncthreads();
        }
      }
    }
  }
#undef MUONH_GLOAD
#undef MUONH_LSTORE

  // ----------------------------------------------------------------- epilogue
  // The fp32 tile goes through LDS in slabs of SLAB rows, stored with its
  // 16-byte granules XOR-swizzled by (row / 8) so that the accumulator
  // writes, the row reads (one granule per lane) and the column reads (8 rows
  // per lane) avoid bank conflicts.  Outputs are then written with
  // row-contiguous accesses: a row pass (X, x32, A, B, O in X orientation)
  // and a column pass (X^T for G3, O when the caller's layout is transposed,
  // and the mirrored tile of the symmetric A and B).
  float* Ct = reinterpret_cast<float*>(smem);
  constexpr int GPR = BN / 4;  // granules per tile row
  static_assert(GPR >= 16, "swizzle needs 16 granules per row");
  auto cidx = [](int rl, int cl) -> int { return rl * BN + ((((cl >> 2) ^ ((rl >> 3) & 15))) << 2) + (cl & 3); };

  double sig = 1.0;
  if (args.first) {
    const double n2 = args.st.sums[2 * u.norm_slot];
    sig = 1.0 / (sqrt(n2) + (double)args.eps);
  }
  const int r = u.r;
  float osq = 0.f;
  const bool mirror = (PHASE != kG3) && (job.tm != job.tn);  // symmetric outputs: also write the transpose
  const bool col_pass = (PHASE == kG3) ? (!args.last || u.o_trans) : mirror;
  constexpr int ROWS_PER_IT = kThreads / GPR;    // row pass: one granule (4 values) per thread
  constexpr int RB = SLAB / ROWS_PER_IT;         // row-pass iterations per slab (all batched)
  constexpr int CPC = SLAB / 8;                  // column pass: 8-row chunks per slab column
  constexpr int COLS_PER_IT = kThreads / CPC;
  static_assert(SLAB % ROWS_PER_IT == 0 && kThreads % CPC == 0 && BN % COLS_PER_IT == 0, "epilogue shape");
  const int gran = tid % GPR, rsub = tid / GPR;
  const int q = tid % CPC, csub = tid / CPC;
  const bool o_vec = (u.o_dtype == DT_BF16) ? ((u.o_ld % 8) == 0 && ((uintptr_t)u.o_ptr % 16) == 0)
                                            : ((u.o_ld % 4) == 0 && ((uintptr_t)u.o_ptr % 16) == 0);
  T* const out12 = reinterpret_cast<T*>(PHASE == kG1 ? u.a : u.b);

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
          const int rl = rbase - sl * SLAB + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          const int cl = wn * WN + j * 32 + (lane & 31);
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
        // G3: X(row, col) <- acc = a X + B X (times sig on the first iteration)
        if (grow < r && gcol < u.ld_s) {
          const int64_t xi = (int64_t)grow * u.ld_s + gcol;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float t = v[e];
            if (args.first) t = (float)((double)t * sig);
            v[e] = (gcol + e < u.s) ? t : 0.f;
          }
          if (!args.last) {
            store4(reinterpret_cast<T*>(u.x), xi, v);
            if (u.x32 != nullptr) store4(u.x32, xi, v);
          } else if (!u.o_trans && grow < u.o_rows) {
            const int nv = min(4, u.o_cols - gcol);
            if (nv > 0) osq += store_out4(u.o_ptr, (int64_t)grow * u.o_ld + gcol, v, nv, u.o_dtype, o_vec);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = 0.f;  // rows >= r: zero padding of X^T
        }
      }
      if (col_pass) *reinterpret_cast<float4*>(cp) = make_float4(v[0], v[1], v[2], v[3]);
    }

    // ---- column pass: tile column cl, 8 slab rows per chunk
    if (col_pass) {
      __syncthreads();
#pragma unroll 2
      for (int it = 0; it < BN / COLS_PER_IT; ++it) {
        const int cl = it * COLS_PER_IT + csub;
        const int gn = col0 + cl;
        const int gi = row0 + sl * SLAB + q * 8;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = Ct[cidx(q * 8 + e, cl)];
        if (PHASE == kG1 || PHASE == kG2) {
          // mirrored tile: row gn of A (or B), columns gi..gi+7
          if (gn < r && gi < u.ld_r) store8(out12, (int64_t)gn * u.ld_r + gi, v);
        } else if (!args.last) {
          if (gn < u.s && gi < u.ld_r) store8(reinterpret_cast<T*>((args.cur ? u.xt[0] : u.xt[1])), (int64_t)gn * u.ld_r + gi, v);
        } else if (gn < u.o_cols && gi < u.o_rows) {
          osq += store_out8(u.o_ptr, (int64_t)gn * u.o_ld + gi, v, min(8, u.o_rows - gi), u.o_dtype, o_vec);
        }
      }
    }
  }
  if (PHASE == kG3 && args.last) {
    block_partial2<kThreads>((double)osq, 0.0, args.st, u.onorm_slot,
                             u.onorm_part0 + job.tm * u.g3_cols + job.tn);
  }
}

// ---------------------------------------------------------------------------
// host launcher
// ---------------------------------------------------------------------------
// Tile configurations (planner.h): 0 = 128 x 128, BK 64; 1 = 256 x 256, BK 64
// (bf16 operands); 2 = 128 x 128, BK 32 (smaller LDS footprint, more blocks
// per CU).  fp32 operands always use 128 x 128 with BK 32.
hipError_t launch_ns_gemm(int op_dt, int phase, int cfg, const NsUnit* units, const GemmJob* jobs, int njobs,
                          float a, float b, float c, float eps, int first, int last, int cur, int no_mma,
                          const SlotTable& st, hipStream_t s) {
  if (njobs <= 0) return hipSuccess;
  NsIterArgs args{a, b, c, eps, first, last, cur, no_mma, njobs, st};
  dim3 grid(njobs), block(kThreads);
#define MUONH_LAUNCH(T, PH, B, K) hipLaunchKernelGGL((k_ns_gemm<T, PH, B, B, K>), grid, block, 0, s, units, jobs, args)
#define MUONH_PHASES(T, B, K)                          \
  do {                                                 \
    if (phase == kG1) MUONH_LAUNCH(T, kG1, B, K);      \
    else if (phase == kG2) MUONH_LAUNCH(T, kG2, B, K); \
    else MUONH_LAUNCH(T, kG3, B, K);                   \
  } while (0)
  if (op_dt == DT_BF16) {
    if (cfg == 1) MUONH_PHASES(bf16_t, 256, 64);
    else if (cfg == 2) MUONH_PHASES(bf16_t, 128, 32);
    else MUONH_PHASES(bf16_t, 128, 64);
  } else {
    MUONH_PHASES(float, 128, 32);
  }
#undef MUONH_PHASES
#undef MUONH_LAUNCH
  return hipGetLastError();
}

}  // namespace muonh
