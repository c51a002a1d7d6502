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
// operand is ever transposed on load.
//
// A launch covers every unit (matrix or HiMuon tile) of a chunk through a job
// list of BM x BN output tiles; job order is remapped so that the jobs one XCD
// runs are contiguous in the list (operand panels shared in its L2).
// Operands are bf16 (v_mfma_f32_32x32x16_bf16) or fp32
// (v_mfma_f32_32x32x2_f32), accumulation is fp32, LDS stages are double
// buffered with a register prefetch of the next stage.
#include "common.h"

namespace muonh {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

template <typename T> struct Mf;
template <> struct Mf<bf16_t> {
  static constexpr int BK = 64;      // K per LDS stage
  static constexpr int KSTEP = 16;   // K per MFMA
  static constexpr int VEC = 8;      // elements per 16-byte chunk
  static constexpr int LDK = BK + 8; // padded LDS row, elements
  using frag = bf16x8_t;
  static __device__ __forceinline__ frag ld(const bf16_t* p) { return *reinterpret_cast<const bf16x8_t*>(p); }
  static __device__ __forceinline__ f32x16_t mma(frag a, frag b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mf<float> {
  static constexpr int BK = 32;
  static constexpr int KSTEP = 2;
  static constexpr int VEC = 4;
  static constexpr int LDK = BK + 4;
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

// Block tile BM x BN, 4 waves in 2 x 2, each wave (BM/2) x (BN/2) built from
// 32 x 32 MFMA tiles.
template <typename T, int PHASE, int BM, int BN>
__global__ __launch_bounds__(kThreads) void k_ns_gemm(const NsUnit* __restrict__ units,
                                                     const GemmJob* __restrict__ jobs, NsIterArgs args) {
  using M = Mf<T>;
  constexpr int BK = M::BK, LDK = M::LDK, VEC = M::VEC, KSTEP = M::KSTEP;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int MI = WM / 32, NI = WN / 32;
  constexpr int CPR = BK / VEC;                          // 16-byte chunks per row
  constexpr int P_LOADS = BM * CPR / kThreads;           // per thread per stage
  constexpr int Q_LOADS = BN * CPR / kThreads;
  static_assert(BM * CPR % kThreads == 0 && BN * CPR % kThreads == 0, "tile/thread mismatch");

  // Main loop: P and Q stages (double buffered).  Epilogue: the fp32 output
  // tile, pitch BN + 1 floats (conflict-free column reads).
  constexpr int kStageBytes = 2 * (BM + BN) * LDK * (int)sizeof(T);
  constexpr int CP = BN + 1;
  constexpr int kTileBytes = BM * CP * 4;
  constexpr int kSmem = kStageBytes > kTileBytes ? kStageBytes : kTileBytes;
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
    P = reinterpret_cast<const T*>(u.b); Q = reinterpret_cast<const T*>(u.xt[args.cur]);
    ldP = u.ld_r; ldQ = u.ld_r; Prows = u.r; Qrows = u.s; K = u.ld_r;
  }
  const int row0 = job.tm * BM, col0 = job.tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  f32x16_t acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nstage = args.no_mma ? 0 : K / BK;
  uint4 pre_p[P_LOADS], pre_q[Q_LOADS];

  auto gload = [&](int ks) {
    const int k0 = ks * BK;
#pragma unroll
    for (int l = 0; l < P_LOADS; ++l) {
      const int c = (tid + l * kThreads) % CPR, r = (tid + l * kThreads) / CPR;
      const int gr = row0 + r;
      pre_p[l] = gr < Prows ? *reinterpret_cast<const uint4*>(P + (int64_t)gr * ldP + k0 + c * VEC)
                            : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int l = 0; l < Q_LOADS; ++l) {
      const int c = (tid + l * kThreads) % CPR, r = (tid + l * kThreads) / CPR;
      const int gr = col0 + r;
      pre_q[l] = gr < Qrows ? *reinterpret_cast<const uint4*>(Q + (int64_t)gr * ldQ + k0 + c * VEC)
                            : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int l = 0; l < P_LOADS; ++l) {
      const int c = (tid + l * kThreads) % CPR, r = (tid + l * kThreads) / CPR;
      *reinterpret_cast<uint4*>(&sP[buf][r * LDK + c * VEC]) = pre_p[l];
    }
#pragma unroll
    for (int l = 0; l < Q_LOADS; ++l) {
      const int c = (tid + l * kThreads) % CPR, r = (tid + l * kThreads) / CPR;
      *reinterpret_cast<uint4*>(&sQ[buf][r * LDK + c * VEC]) = pre_q[l];
    }
  };

  if (nstage > 0) {
    gload(0);
    lstore(0);
    __syncthreads();
    for (int ks = 0; ks < nstage; ++ks) {
      const int buf = ks & 1;
      if (ks + 1 < nstage) gload(ks + 1);
      const T* sp = sP[buf];
      const T* sq = sQ[buf];
#pragma unroll
      for (int kk = 0; kk < BK; kk += KSTEP) {
        const int koff = kk + (lane >> 5) * (KSTEP / 2);
        typename M::frag fa[MI], fb[NI];
#pragma unroll
        for (int i = 0; i < MI; ++i) fa[i] = M::ld(sp + (wm * WM + i * 32 + (lane & 31)) * LDK + koff);
#pragma unroll
        for (int j = 0; j < NI; ++j) fb[j] = M::ld(sq + (wn * WN + j * 32 + (lane & 31)) * LDK + koff);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NI; ++j) acc[i][j] = M::mma(fa[i], fb[j], acc[i][j]);
      }
      if (ks + 1 < nstage) {
        lstore(buf ^ 1);
        __syncthreads();
      }
    }
  }

  // ----------------------------------------------------------------- epilogue
  // Stage the fp32 tile in LDS, then write every output with 16-byte,
  // row-contiguous accesses: a row pass (X, x32, A, B, O in X orientation) and,
  // for G3, a column pass (X^T, or O when the caller's layout is transposed).
  __syncthreads();
  float* Ct = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rl = wm * WM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const int cl = wn * WN + j * 32 + (lane & 31);
        Ct[rl * CP + cl] = acc[i][j][v];
      }
  __syncthreads();

  double sig = 1.0;
  if (args.first) {
    const double n2 = args.st.sums[2 * u.norm_slot];
    sig = 1.0 / (sqrt(n2) + (double)args.eps);
  }
  const int r = u.r;
  float osq = 0.f;
  constexpr int CPR_OUT = BN / 8;            // 8-element chunks per tile row
  constexpr int ROWS_PER_IT = kThreads / CPR_OUT;
  const int chunk = tid % CPR_OUT, rsub = tid / CPR_OUT;
  const bool o_vec = (u.o_dtype == DT_BF16) ? ((u.o_ld % 8) == 0 && ((uintptr_t)u.o_ptr % 16) == 0)
                                            : ((u.o_ld % 4) == 0 && ((uintptr_t)u.o_ptr % 16) == 0);

  // ---- row pass
#pragma unroll 1
  for (int it = 0; it < BM / ROWS_PER_IT; ++it) {
    const int rl = it * ROWS_PER_IT + rsub;
    const int grow = row0 + rl;
    const int cl = chunk * 8;
    const int gcol = col0 + cl;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = Ct[rl * CP + cl + e];
    if (PHASE == kG1 || PHASE == kG2) {
      if (grow < r && gcol < u.ld_r) {
        T* out = reinterpret_cast<T*>(PHASE == kG1 ? u.a : u.b);
        const int64_t oi = (int64_t)grow * u.ld_r + gcol;
        if (PHASE == kG1) {
          const float sc = (float)(sig * sig);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = (gcol + e < r) ? v[e] * sc : 0.f;
        } else {
          float a8[8];
          load8(reinterpret_cast<const T*>(u.a), oi, a8);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = (gcol + e < r) ? fmaf(args.c, v[e], args.b * a8[e]) : 0.f;
        }
        store8(out, oi, v);
      }
    } else {
      // G3: X(row, col) <- a X(row, col) + acc (times sig on the first iteration)
      if (grow < r && gcol < u.ld_s) {
        const int64_t xi = (int64_t)grow * u.ld_s + gcol;
        float prev[8];
        if (!args.first && u.x32 != nullptr) load8(u.x32, xi, prev);
        else load8(reinterpret_cast<const T*>(u.x), xi, prev);
        const float a = args.no_mma ? 1.f : args.a;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float t = fmaf(a, prev[e], v[e]);
          if (args.first) t = (float)((double)t * sig);
          v[e] = (gcol + e < u.s) ? t : 0.f;
        }
        if (!args.last) {
          store8(reinterpret_cast<T*>(u.x), xi, v);
          if (u.x32 != nullptr) store8(u.x32, xi, v);
        } else if (!u.o_trans && grow < u.o_rows) {
          const int nv = min(8, u.o_cols - gcol);
          if (nv > 0) {
            const int64_t oi = (int64_t)grow * u.o_ld + gcol;
            if (o_vec && nv == 8) {
              float rv[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) rv[e] = (u.o_dtype == DT_BF16) ? St<bf16_t>::round(v[e]) : v[e];
              if (u.o_dtype == DT_BF16) store8(reinterpret_cast<bf16_t*>(u.o_ptr), oi, rv);
              else store8(reinterpret_cast<float*>(u.o_ptr), oi, rv);
#pragma unroll
              for (int e = 0; e < 8; ++e) osq = fmaf(rv[e], rv[e], osq);
            } else {
              for (int e = 0; e < nv; ++e) {
                const float sv = store_dyn(u.o_ptr, oi + e, v[e], u.o_dtype);
                osq = fmaf(sv, sv, osq);
              }
            }
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.f;  // rows >= r: zero padding of X^T
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) Ct[rl * CP + cl + e] = v[e];
    }
  }

  if (PHASE == kG3 && (!args.last || u.o_trans)) {
    __syncthreads();
    // ---- column pass: tile column cl -> X^T row (col0 + cl), 8 rows per chunk
    T* XT = reinterpret_cast<T*>(u.xt[args.cur ^ 1]);
    constexpr int CPC = BM / 8;                 // 8-row chunks per tile column
    constexpr int COLS_PER_IT = kThreads / CPC;
    const int q = tid % CPC, csub = tid / CPC;
#pragma unroll 1
    for (int it = 0; it < BN / COLS_PER_IT; ++it) {
      const int cl = it * COLS_PER_IT + csub;
      const int gn = col0 + cl;
      const int gi = row0 + q * 8;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = Ct[(q * 8 + e) * CP + cl];
      if (!args.last) {
        if (gn < u.s && gi < u.ld_r) store8(XT, (int64_t)gn * u.ld_r + gi, v);
      } else if (gn < u.o_cols && gi < u.o_rows) {
        const int nv = min(8, u.o_rows - gi);
        const int64_t oi = (int64_t)gn * u.o_ld + gi;
        if (o_vec && nv == 8) {
          float rv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) rv[e] = (u.o_dtype == DT_BF16) ? St<bf16_t>::round(v[e]) : v[e];
          if (u.o_dtype == DT_BF16) store8(reinterpret_cast<bf16_t*>(u.o_ptr), oi, rv);
          else store8(reinterpret_cast<float*>(u.o_ptr), oi, rv);
#pragma unroll
          for (int e = 0; e < 8; ++e) osq = fmaf(rv[e], rv[e], osq);
        } else {
          for (int e = 0; e < nv; ++e) {
            const float sv = store_dyn(u.o_ptr, oi + e, v[e], u.o_dtype);
            osq = fmaf(sv, sv, osq);
          }
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
constexpr int kBM = 128, kBN = 128;

int gemm_tile_m() { return kBM; }
int gemm_tile_n() { return kBN; }

hipError_t launch_ns_gemm(int op_dt, int phase, const NsUnit* units, const GemmJob* jobs, int njobs,
                          float a, float b, float c, float eps, int first, int last, int cur, int no_mma,
                          const SlotTable& st, hipStream_t s) {
  if (njobs <= 0) return hipSuccess;
  NsIterArgs args{a, b, c, eps, first, last, cur, no_mma, njobs, st};
  dim3 grid(njobs), block(kThreads);
#define MUONH_LAUNCH(T, PH) hipLaunchKernelGGL((k_ns_gemm<T, PH, kBM, kBN>), grid, block, 0, s, units, jobs, args)
  if (op_dt == DT_BF16) {
    if (phase == kG1) MUONH_LAUNCH(bf16_t, kG1);
    else if (phase == kG2) MUONH_LAUNCH(bf16_t, kG2);
    else MUONH_LAUNCH(bf16_t, kG3);
  } else {
    if (phase == kG1) MUONH_LAUNCH(float, kG1);
    else if (phase == kG2) MUONH_LAUNCH(float, kG2);
    else MUONH_LAUNCH(float, kG3);
  }
#undef MUONH_LAUNCH
  return hipGetLastError();
}

}  // namespace muonh
