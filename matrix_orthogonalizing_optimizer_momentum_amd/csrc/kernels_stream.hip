// HBM-streaming kernels of the MuonH step (gfx950):
//   k_momentum_prep  M <- beta*M + G (Muon explainer, momentum recap /
//                    Equation 1), the Frobenius sum of squares of the stored M
//                    per Newton-Schulz unit, and X0^T written into the
//                    unit's workspace (the wide-side orientation of the
//                    Muon explainer's code section is a layout choice here,
//                    never a copy of its own);
//   k_hook_reduce    pass 1 of the Hyperball / RadialBrake / RelativeUpdate
//                    hook: per-matrix sums of ||W'||^2 and ||W||^2 in fp64;
//   k_hook_write     pass 2: re-projection / brake / relative step
//                    (Hyperball show notes, Algorithm 1 and Method; hook PR,
//                    PR description, review summary and the zero-norm review
//                    comments);
//   k_sumsq          per-matrix ||U||^2 for the stand-alone projection;
//   k_adam_moments,  AdamH: Adam's moments and the norms behind its hook,
//   k_adam_write     then the hook on Adam's direction (two passes in all).
// All of them are bandwidth-bound: 16-byte vector accesses, 64x64 blocks
// with an LDS transpose where a layout flips, one deterministic fp64
// reduction commit per block.
#include "common.h"

namespace muonh {

constexpr int kMomThreads = 256;
constexpr int kHookThreads = 256;
constexpr int kHookPerThread = 32;  // elements per thread per block (4 x 8)
static_assert(kHookBlockElems == kHookThreads * kHookPerThread, "hook block size");

// ---------------------------------------------------------------------------
// momentum + norm + X0 layouts
// ---------------------------------------------------------------------------
template <typename ST, typename OT>
__global__ __launch_bounds__(kMomThreads) void k_momentum_prep(
    const MomMat* __restrict__ mats, const MomBlock* __restrict__ blocks,
    const NsUnit* __restrict__ units, SlotTable st, float beta, float gcoef, int nesterov) {
  __shared__ float tile[64][65];
  const MomBlock blk = blocks[blockIdx.x];
  const MomMat mm = mats[blk.mat];
  const int t = threadIdx.x;
  const int cc = t & 7;   // 8-element column chunk
  const int rr = t >> 3;  // 0..31
  const int64_t H = mm.H, W = mm.W;
  const bool vec = (W % 8) == 0;
  const ST* __restrict__ g = reinterpret_cast<const ST*>(mm.g);
  ST* __restrict__ m = reinterpret_cast<ST*>(mm.m);

  // Issue both rows' loads before any store (m is read and written), and
  // before any value is converted (a conversion next to its load makes the
  // compiler wait for it there).
  Raw8<ST> gr[2], mr[2];
  bool fast[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int64_t row = (int64_t)blk.br * 64 + rr + 32 * p;
    const int64_t col0 = (int64_t)blk.bc * 64 + cc * 8;
    fast[p] = row < H && vec && col0 + 8 <= W;
    if (fast[p]) gr[p].load(g, row * W + col0);
  }
  if (m != nullptr) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int64_t row = (int64_t)blk.br * 64 + rr + 32 * p;
      const int64_t col0 = (int64_t)blk.bc * 64 + cc * 8;
      if (fast[p]) mr[p].load(m, row * W + col0);
    }
  }
  float sq = 0.f;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int lr = rr + 32 * p;
    const int64_t row = (int64_t)blk.br * 64 + lr;
    const int64_t col0 = (int64_t)blk.bc * 64 + cc * 8;
    // v: the stored buffer; the NS input is v, or the Nesterov blend
    // gcoef*G + beta*v (Muon explainer, code section)
    float v[8];
    if (fast[p]) {
      float gv[8];
      gr[p].unpack(gv);
      if (m != nullptr) {
        float mv[8];
        mr[p].unpack(mv);
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = St<ST>::round(fmaf(beta, mv[k], gcoef * gv[k]));
        store8(m, row * W + col0, v);
        if (nesterov) {
#pragma unroll
          for (int k = 0; k < 8; ++k) v[k] = fmaf(beta, v[k], gcoef * gv[k]);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = gv[k];
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int64_t col = col0 + k;
        float x = 0.f;
        if (row < H && col < W) {
          const int64_t idx = row * W + col;
          float gg = St<ST>::ld(g, idx);
          if (m != nullptr) {
            x = St<ST>::round(fmaf(beta, St<ST>::ld(m, idx), gcoef * gg));
            St<ST>::st(m, idx, x);
            if (nesterov) x = fmaf(beta, x, gcoef * gg);
          } else {
            x = gg;
          }
        }
        v[k] = x;
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      sq = fmaf(v[k], v[k], sq);
      tile[lr][cc * 8 + k] = v[k];
    }
  }

  if (mm.write_x) {
    // Destination unit and in-unit coordinates of this block's origin.
    int unit_id = mm.unit0;
    int64_t r0 = (int64_t)blk.br * 64, c0 = (int64_t)blk.bc * 64;  // M coordinates
    if (mm.tile_T > 0) {
      const int T = mm.tile_T;
      unit_id += (int)(r0 / T) * mm.ntc + (int)(c0 / T);
      r0 %= T;
      c0 %= T;
    }
    const NsUnit u = units[unit_id];
    // X0^T into xt[0]: ld_s rows of ld_r.  The block grid spans the padded
    // extent and its values outside the matrix are zero, so the padding is
    // written too.
    OT* const xt = reinterpret_cast<OT*>(u.xt[0]);
    // fp32 X0^T beside it when the NS input is not a bf16 value (fp32 state or
    // the Nesterov blend) and the operands are bf16: the first iteration's
    // a X term is then seeded from it instead of the rounded operand copy
    float* const x32 = mm.write_x32 ? u.x32 : nullptr;
    const int64_t ld = u.ld_r;
    if (mm.trans) {
      // X = M^T: X^T has M's layout; same element positions as loaded.
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int lr = rr + 32 * p;
        const int64_t row = r0 + lr;
        const int64_t col = c0 + cc * 8;
        if (row < u.ld_s && col + 8 <= ld) {
          float v[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) v[k] = tile[lr][cc * 8 + k];
          store8(xt, row * ld + col, v);
          if (x32 != nullptr) store8(x32, row * ld + col, v);
        }
      }
    } else {
      // X = M: X^T row = M column, 16 consecutive M rows per thread.
      __syncthreads();
      const int lc = t >> 2;
      const int seg = (t & 3) * 16;
      const int64_t frow = c0 + lc;
      const int64_t fcol = r0 + seg;
      if (frow < u.ld_s) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (fcol + 8 * h + 8 <= ld) {
            float v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = tile[seg + 8 * h + k][lc];
            store8(xt, frow * ld + fcol + 8 * h, v);
            if (x32 != nullptr) store8(x32, frow * ld + fcol + 8 * h, v);
          }
        }
      }
    }
  }
  if (blk.slot >= 0) block_partial2<kMomThreads>((double)sq, 0.0, st, blk.slot, blk.part);
}

// ---------------------------------------------------------------------------
// hook passes
// ---------------------------------------------------------------------------
__device__ __forceinline__ void load8_dyn(const void* p, int64_t i, int dtype, float (&v)[8]) {
  if (dtype == DT_BF16) load8(reinterpret_cast<const bf16_t*>(p), i, v);
  else load8(reinterpret_cast<const float*>(p), i, v);
}

// The kHookPerThread elements a thread of a whole hook block owns (chunks
// base + (c * kHookThreads + t) * 8), W (fp32) and, when used, O (run-time
// dtype), every load issued before any value is used.
struct HookChunks {
  static constexpr int NC = kHookPerThread / 8;
  Raw8<float> w[NC], of[NC];
  Raw8<bf16_t> ob[NC];
  __device__ __forceinline__ static int64_t at(int64_t base, int c) {
    return base + ((int64_t)c * kHookThreads + threadIdx.x) * 8;
  }
  __device__ __forceinline__ void load(const float* wp, const void* op, int o_dtype, int64_t base) {
#pragma unroll
    for (int c = 0; c < NC; ++c) w[c].load(wp, at(base, c));
    if (op != nullptr) {
      if (o_dtype == DT_BF16) {
#pragma unroll
        for (int c = 0; c < NC; ++c) ob[c].load(reinterpret_cast<const bf16_t*>(op), at(base, c));
      } else {
#pragma unroll
        for (int c = 0; c < NC; ++c) of[c].load(reinterpret_cast<const float*>(op), at(base, c));
      }
    }
  }
  __device__ __forceinline__ void get(int c, bool use_o, int o_dtype, float (&wv)[8], float (&ov)[8]) const {
    w[c].unpack(wv);
    if (!use_o) {
#pragma unroll
      for (int k = 0; k < 8; ++k) ov[k] = 0.f;
    } else if (o_dtype == DT_BF16) {
      ob[c].unpack(ov);
    } else {
      of[c].unpack(ov);
    }
  }
};

// Coefficient applied to O in W' = W - coef * O: eta times the shape scale
// (RadialBrake, plain update), eta / ||O|| times the step scale (Hyperball:
// 1 or rho), eta ||W|| / ||O|| (RelativeUpdate, from pass 1's ||W||^2).
__device__ __forceinline__ float hook_coef(const HookMat& hm, const SlotTable& st, float eta, int mode) {
  if (mode == kModeRB || mode == kModeNone) return eta * hm.oscale;
  if (hm.o == nullptr || hm.onorm_slot < 0) return 0.f;
  const double n2 = st.sums[2 * hm.onorm_slot];
  if (!(n2 > 0.0)) return 0.f;
  if (mode == kModeRel) return (float)((double)eta * sqrt(st.sums[2 * hm.slot + 1]) / sqrt(n2));
  return (float)((double)eta * (double)hm.oscale / sqrt(n2));
}

// ||W - c O||^2 formed as ||W||^2 - 2 c <W, O> + c^2 ||O||^2: rounding can take
// it below zero, which is clamped; a NaN (a non-finite O or W) is kept, so the
// matrix takes the same branch and is counted as non-finite exactly as when
// pass 1 sums ||W - c O||^2 itself.
__device__ __forceinline__ double clamp_expanded(double e) { return e < 0.0 ? 0.0 : e; }

// Per-matrix decision of pass 2, identical in every block of the matrix,
// from ||W'||^2 (v0) and ||W||^2 (v1).  branch 0: scale W', 1: scale W
// (Hyperball restore), 2: leave W.
struct HookDecision {
  int branch;
  double scale;
};
__device__ __forceinline__ HookDecision hook_decide(int mode, double v0, double v1, float rho_f, float zero_rel_eps,
                                                    float outward, float inward, float rb_eps) {
  const double nwp = sqrt(v0), nw = sqrt(v1);
  if (mode == kModeNone || mode == kModeRel) return {0, 1.0};
  if (mode == kModeRB) {
    const double s = (nwp > nw) ? (double)outward : (double)inward;
    if (nwp > (double)rb_eps) return {0, (nw + s * (nwp - nw)) / nwp};
    return {0, 1.0};
  }
  const double rho = (double)rho_f;
  if (nwp >= (double)zero_rel_eps * rho) return {0, rho / nwp};
  if (nw > 0.0) return {1, rho / nw};
  return {2, 1.0};
}

// Device flag counters for one matrix (called once per matrix).
__device__ __forceinline__ void hook_flags(int mode, float coef, bool has_o, int branch, double v0, double v1,
                                           Flags* flags) {
  if (flags == nullptr) return;
  if ((mode == kModeHB || mode == kModeRel) && coef == 0.f && has_o) atomicAdd(&flags->zero_update, 1ull);
  if (mode == kModeHB) {
    if (branch == 1) atomicAdd(&flags->restored, 1ull);
    if (branch == 2) atomicAdd(&flags->unrestorable, 1ull);
  }
  if (!isfinite(v0) || !isfinite(v1)) atomicAdd(&flags->nonfinite, 1ull);
}

template <int MODE>
__global__ __launch_bounds__(kHookThreads) void k_hook_reduce(
    const HookMat* __restrict__ mats, const HookBlock* __restrict__ blocks, SlotTable st, float eta) {
  const HookBlock hb = blocks[blockIdx.x];
  const HookMat hm = mats[hb.mat];
  // RelativeUpdate needs only ||W||^2 here (its coefficient depends on it).
  const float coef = MODE == kModeRel ? 0.f : hook_coef(hm, st, eta, MODE);
  const void* const op = MODE == kModeRel ? nullptr : hm.o;
  double s0 = 0.0, s1 = 0.0;
  const int64_t base = (int64_t)hb.blk * kHookBlockElems;
  auto add = [&](const float (&w)[8], const float (&o)[8]) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float wp = fmaf(-coef, o[k], w[k]);
      s0 = fma((double)wp, (double)wp, s0);
      s1 = fma((double)w[k], (double)w[k], s1);
    }
  };
  if (base + kHookBlockElems <= hm.numel) {  // a whole block: all loads in flight together
    HookChunks ch;
    ch.load(hm.w, op, hm.o_dtype, base);
#pragma unroll
    for (int c = 0; c < HookChunks::NC; ++c) {
      float w[8], o[8];
      ch.get(c, op != nullptr, hm.o_dtype, w, o);
      add(w, o);
    }
  } else {
    for (int it = 0; it < kHookPerThread / 8; ++it) {
      const int64_t i = HookChunks::at(base, it);
      if (i >= hm.numel) break;
      float w[8], o[8];
      if (i + 8 <= hm.numel) {
        load8(hm.w, i, w);
        if (op) load8_dyn(op, i, hm.o_dtype, o);
        else for (int k = 0; k < 8; ++k) o[k] = 0.f;
      } else {
        for (int k = 0; k < 8; ++k) {
          const bool ok = i + k < hm.numel;
          w[k] = ok ? hm.w[i + k] : 0.f;
          o[k] = (ok && op) ? load_dyn(op, i + k, hm.o_dtype) : 0.f;
        }
      }
      add(w, o);
    }
  }
  block_partial2<kHookThreads>(s0, s1, st, hm.slot, hb.blk);
}

// Per matrix: when HookMat::fused is set, the producer of O summed <W, O>
// (second value of the O-norm slot) and ||W||^2 (second value of the hook
// slot) at its store, and ||W - coef O||^2 is expanded as
// ||W||^2 - 2 coef <W, O> + coef^2 ||O||^2 in fp64; otherwise pass 1
// (k_hook_reduce) summed ||W'||^2 and ||W||^2.
template <int MODE>
__global__ __launch_bounds__(kHookThreads) void k_hook_write(
    const HookMat* __restrict__ mats, const HookBlock* __restrict__ blocks, SlotTable st, float eta,
    float zero_rel_eps, float outward, float inward, float rb_eps, float decay, Flags* flags) {
  const HookBlock hb = blocks[blockIdx.x];
  const HookMat hm = mats[hb.mat];
  const float coef = hook_coef(hm, st, eta, MODE);
  double v0 = 0.0, v1 = 0.0;  // ||W'||^2, ||W||^2 (none for Muon's own update)
  if (MODE != kModeNone) {
    v1 = st.sums[2 * hm.slot + 1];
    if (hm.fused) {
      const double c = (double)coef;
      const double uu = hm.onorm_slot >= 0 ? st.sums[2 * hm.onorm_slot] : 0.0;
      const double wo = hm.onorm_slot >= 0 ? st.sums[2 * hm.onorm_slot + 1] : 0.0;
      v0 = clamp_expanded(v1 - 2.0 * c * wo + c * c * uu);
    } else {
      v0 = st.sums[2 * hm.slot];
    }
  }
  const HookDecision dec = hook_decide(MODE, v0, v1, hm.rho, zero_rel_eps, outward, inward, rb_eps);
  const int branch = dec.branch;
  const double scale = dec.scale;
  if (hb.blk == 0 && threadIdx.x == 0) hook_flags(MODE, coef, hm.o != nullptr, branch, v0, v1, flags);
  if (branch == 2) return;
  const int64_t base = (int64_t)hb.blk * kHookBlockElems;
  const bool use_o = hm.o != nullptr && branch == 0;
  auto apply = [&](const float (&w)[8], const float (&o)[8], float (&r)[8]) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (MODE == kModeNone) {
        // Muon explainer, code section: decoupled decay, then W - eta * O'
        r[k] = fmaf(-coef, o[k], w[k] * decay);
      } else if (MODE == kModeRel) {
        r[k] = fmaf(-coef, o[k], w[k]);
      } else {
        const float base_v = (branch == 0) ? fmaf(-coef, o[k], w[k]) : w[k];
        r[k] = (float)((double)base_v * scale);
      }
    }
  };
  if (base + kHookBlockElems <= hm.numel) {  // a whole block: all loads in flight together
    HookChunks ch;
    ch.load(hm.w, use_o ? hm.o : nullptr, hm.o_dtype, base);
#pragma unroll
    for (int c = 0; c < HookChunks::NC; ++c) {
      float w[8], o[8], r[8];
      ch.get(c, use_o, hm.o_dtype, w, o);
      apply(w, o, r);
      store8(hm.w, HookChunks::at(base, c), r);
    }
    return;
  }
  for (int it = 0; it < kHookPerThread / 8; ++it) {
    const int64_t i = HookChunks::at(base, it);
    if (i >= hm.numel) break;
    float w[8], o[8];
    const bool full = i + 8 <= hm.numel;
    if (full) {
      load8(hm.w, i, w);
      if (use_o) load8_dyn(hm.o, i, hm.o_dtype, o);
      else for (int k = 0; k < 8; ++k) o[k] = 0.f;
    } else {
      for (int k = 0; k < 8; ++k) {
        const bool ok = i + k < hm.numel;
        w[k] = ok ? hm.w[i + k] : 0.f;
        o[k] = (ok && use_o) ? load_dyn(hm.o, i + k, hm.o_dtype) : 0.f;
      }
    }
    float r[8];
    apply(w, o, r);
    if (full) {
      store8(hm.w, i, r);
    } else {
      for (int k = 0; k < 8; ++k)
        if (i + k < hm.numel) hm.w[i + k] = r[k];
    }
  }
}

// ---------------------------------------------------------------------------
// AdamH (Hyperball show notes, Method: the wrapper around Adam's
// preconditioned update; Muon explainer, Equation 2 text for Adam itself)
// ---------------------------------------------------------------------------
// Adam's direction for one element from the updated moments.
__device__ __forceinline__ float adam_u(float m, float v, const AdamArgs& a) {
  return (m * a.ibc1) / (sqrtf(v * a.ibc2) + a.eps);
}

// Pass 1: the moment updates (stored in place) and, per matrix, ||U||^2,
// <W, U> and ||W||^2 in fp64, from which pass 2 gets ||W - coef U||^2
// without a pass of its own (the plain AdamW update needs none of them).
template <typename GT, bool SUMS>
__global__ __launch_bounds__(kHookThreads) void k_adam_moments(
    const HookMat* __restrict__ mats, const HookBlock* __restrict__ blocks, SlotTable st, AdamArgs a) {
  const HookBlock hb = blocks[blockIdx.x];
  const HookMat hm = mats[hb.mat];
  const GT* const g = reinterpret_cast<const GT*>(hm.o);
  const float c1 = 1.f - a.b1, c2 = 1.f - a.b2;
  double s_uu = 0.0, s_wu = 0.0, s_ww = 0.0;
  const int64_t base = (int64_t)hb.blk * kHookBlockElems;
  auto update = [&](float (&gv)[8], float (&m)[8], float (&v)[8], const float (&w)[8]) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      m[k] = fmaf(a.b1, m[k], c1 * gv[k]);
      v[k] = fmaf(a.b2, v[k], c2 * (gv[k] * gv[k]));
      if (SUMS) {
        const double u = (double)adam_u(m[k], v[k], a), wd = (double)w[k];
        s_uu = fma(u, u, s_uu);
        s_wu = fma(wd, u, s_wu);
        s_ww = fma(wd, wd, s_ww);
      }
    }
  };
  constexpr int NC = kHookPerThread / 8;
  if (base + kHookBlockElems <= hm.numel) {  // a whole block: every chunk's loads in flight together
    Raw8<GT> gr[NC];
    Raw8<float> mr[NC], vr[NC], wr[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int64_t i = HookChunks::at(base, c);
      gr[c].load(g, i);
      mr[c].load(hm.am, i);
      vr[c].load(hm.av, i);
      if (SUMS) wr[c].load(hm.w, i);
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int64_t i = HookChunks::at(base, c);
      float gv[8], m[8], v[8], w[8];
      gr[c].unpack(gv);
      mr[c].unpack(m);
      vr[c].unpack(v);
      if (SUMS) wr[c].unpack(w);
      else for (int k = 0; k < 8; ++k) w[k] = 0.f;
      update(gv, m, v, w);
      store8(hm.am, i, m);
      store8(hm.av, i, v);
    }
  } else {
    for (int it = 0; it < NC; ++it) {
      const int64_t i = HookChunks::at(base, it);
      if (i >= hm.numel) break;
      const bool full = i + 8 <= hm.numel;
      float gv[8], m[8], v[8], w[8];
      if (full) {
        load8(g, i, gv);
        load8(hm.am, i, m);
        load8(hm.av, i, v);
        if (SUMS) load8(hm.w, i, w);
        else for (int k = 0; k < 8; ++k) w[k] = 0.f;
      } else {
        for (int k = 0; k < 8; ++k) {
          const bool ok = i + k < hm.numel;
          gv[k] = ok ? load_dyn(g, i + k, hm.o_dtype) : 0.f;
          m[k] = ok ? hm.am[i + k] : 0.f;
          v[k] = ok ? hm.av[i + k] : 0.f;
          w[k] = (ok && SUMS) ? hm.w[i + k] : 0.f;
        }
      }
      update(gv, m, v, w);
      if (full) {
        store8(hm.am, i, m);
        store8(hm.av, i, v);
      } else {
        for (int k = 0; k < 8; ++k)
          if (i + k < hm.numel) { hm.am[i + k] = m[k]; hm.av[i + k] = v[k]; }
      }
    }
  }
  if (!SUMS) return;
  constexpr int NW = kHookThreads / 64;
  __shared__ double red[3][NW];
  const int wv = threadIdx.x >> 6;
  s_uu = wave_sum(s_uu);
  s_wu = wave_sum(s_wu);
  s_ww = wave_sum(s_ww);
  if ((threadIdx.x & 63) == 0) { red[0][wv] = s_uu; red[1][wv] = s_wu; red[2][wv] = s_ww; }
  __syncthreads();
  if (threadIdx.x == 0) {
    double t0 = 0.0, t1 = 0.0, t2 = 0.0;
#pragma unroll
    for (int q = 0; q < NW; ++q) { t0 += red[0][q]; t1 += red[1][q]; t2 += red[2][q]; }
    const int64_t pa = st.part_base[hm.onorm_slot] + hb.blk, pb = st.part_base[hm.slot] + hb.blk;
    gmem(st.partials)[2 * pa] = t0;
    gmem(st.partials)[2 * pa + 1] = t1;
    gmem(st.partials)[2 * pb] = 0.0;
    gmem(st.partials)[2 * pb + 1] = t2;
  }
}

// Pass 2: the hook applied to Adam's direction, recomputed from the stored
// moments (bitwise the values pass 1 summed).  ||W - coef U||^2 is expanded as
// ||W||^2 - 2 coef <W, U> + coef^2 ||U||^2 in fp64.
template <int MODE>
__global__ __launch_bounds__(kHookThreads) void k_adam_write(
    const HookMat* __restrict__ mats, const HookBlock* __restrict__ blocks, SlotTable st, AdamArgs a, float eta,
    float zero_rel_eps, float outward, float inward, float rb_eps, float decay, Flags* flags) {
  const HookBlock hb = blocks[blockIdx.x];
  const HookMat hm = mats[hb.mat];
  float coef = eta;
  double v0 = 0.0, v1 = 0.0;
  if (MODE != kModeNone) {
    const double uu = st.sums[2 * hm.onorm_slot], wu = st.sums[2 * hm.onorm_slot + 1];
    v1 = st.sums[2 * hm.slot + 1];
    if (MODE == kModeHB) coef = uu > 0.0 ? (float)((double)eta * (double)hm.oscale / sqrt(uu)) : 0.f;
    else if (MODE == kModeRel) coef = uu > 0.0 ? (float)((double)eta * sqrt(v1) / sqrt(uu)) : 0.f;
    const double c = (double)coef;
    v0 = clamp_expanded(v1 - 2.0 * c * wu + c * c * uu);
  }
  const HookDecision dec = hook_decide(MODE, v0, v1, hm.rho, zero_rel_eps, outward, inward, rb_eps);
  if (hb.blk == 0 && threadIdx.x == 0) hook_flags(MODE, coef, true, dec.branch, v0, v1, flags);
  if (dec.branch == 2) return;
  const int64_t base = (int64_t)hb.blk * kHookBlockElems;
  auto apply = [&](const float (&w)[8], const float (&m)[8], const float (&v)[8], float (&r)[8]) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float u = adam_u(m[k], v[k], a);
      if (MODE == kModeNone) {
        r[k] = fmaf(-coef, u, w[k] * decay);  // AdamW: decoupled decay, then W - eta U
      } else if (MODE == kModeRel) {
        r[k] = fmaf(-coef, u, w[k]);
      } else {
        const float base_v = (dec.branch == 0) ? fmaf(-coef, u, w[k]) : w[k];
        r[k] = (float)((double)base_v * dec.scale);
      }
    }
  };
  constexpr int NC = kHookPerThread / 8;
  if (base + kHookBlockElems <= hm.numel) {  // a whole block: every chunk's loads in flight together
    Raw8<float> wr[NC], mr[NC], vr[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int64_t i = HookChunks::at(base, c);
      wr[c].load(hm.w, i);
      mr[c].load(hm.am, i);
      vr[c].load(hm.av, i);
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float w[8], m[8], v[8], r[8];
      wr[c].unpack(w);
      mr[c].unpack(m);
      vr[c].unpack(v);
      apply(w, m, v, r);
      store8(hm.w, HookChunks::at(base, c), r);
    }
    return;
  }
  for (int it = 0; it < NC; ++it) {
    const int64_t i = HookChunks::at(base, it);
    if (i >= hm.numel) break;
    const bool full = i + 8 <= hm.numel;
    float w[8], m[8], v[8];
    if (full) {
      load8(hm.w, i, w);
      load8(hm.am, i, m);
      load8(hm.av, i, v);
    } else {
      for (int k = 0; k < 8; ++k) {
        const bool ok = i + k < hm.numel;
        w[k] = ok ? hm.w[i + k] : 0.f;
        m[k] = ok ? hm.am[i + k] : 0.f;
        v[k] = ok ? hm.av[i + k] : 1.f;
      }
    }
    float r[8];
    apply(w, m, v, r);
    if (full) {
      store8(hm.w, i, r);
    } else {
      for (int k = 0; k < 8; ++k)
        if (i + k < hm.numel) hm.w[i + k] = r[k];
    }
  }
}

// ||U||^2 per matrix (HookMat.o is U; the result lands in slot onorm_slot).
__global__ __launch_bounds__(kHookThreads) void k_sumsq(
    const HookMat* __restrict__ mats, const HookBlock* __restrict__ blocks, SlotTable st) {
  const HookBlock hb = blocks[blockIdx.x];
  const HookMat hm = mats[hb.mat];
  if (hm.o == nullptr || hm.onorm_slot < 0) return;  // zero update: no norm needed (uniform per block)
  double s0 = 0.0;
  const int64_t base = (int64_t)hb.blk * kHookBlockElems;
  for (int it = 0; it < kHookPerThread / 8; ++it) {
    const int64_t i = base + ((int64_t)it * kHookThreads + threadIdx.x) * 8;
    if (i >= hm.numel) break;
    float o[8];
    if (i + 8 <= hm.numel) {
      load8_dyn(hm.o, i, hm.o_dtype, o);
    } else {
      for (int k = 0; k < 8; ++k) o[k] = (i + k < hm.numel) ? load_dyn(hm.o, i + k, hm.o_dtype) : 0.f;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) s0 = fma((double)o[k], (double)o[k], s0);
  }
  block_partial2<kHookThreads>(s0, 0.0, st, hm.onorm_slot, hb.blk);
}

// Sum each slot's partials in a fixed order: slots [slot0, slot0 + gridDim.x).
__global__ __launch_bounds__(256) void k_finalize(SlotTable st, int slot0) {
  const int slot = slot0 + blockIdx.x;
  const int n = st.nparts[slot];
  const int64_t base = st.part_base[slot];
  double t0 = 0.0, t1 = 0.0;
  for (int i = threadIdx.x; i < n; i += 256) {
    t0 += st.partials[2 * (base + i)];
    t1 += st.partials[2 * (base + i) + 1];
  }
  __shared__ double red[2][4];
  t0 = wave_sum(t0);
  t1 = wave_sum(t1);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { red[0][w] = t0; red[1][w] = t1; }
  __syncthreads();
  if (threadIdx.x == 0) {
    st.sums[2 * slot] = ((red[0][0] + red[0][1]) + red[0][2]) + red[0][3];
    st.sums[2 * slot + 1] = ((red[1][0] + red[1][1]) + red[1][2]) + red[1][3];
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
hipError_t launch_momentum_prep(int state_dt, int op_dt, const MomMat* mats, const MomBlock* blocks,
                                int nblocks, const NsUnit* units, const SlotTable& st, float beta,
                                float gcoef, int nesterov, hipStream_t s) {
  if (nblocks <= 0) return hipSuccess;
  dim3 grid(nblocks), block(kMomThreads);
#define MUONH_MOM(ST, OT) \
  hipLaunchKernelGGL((k_momentum_prep<ST, OT>), grid, block, 0, s, mats, blocks, units, st, beta, gcoef, nesterov)
  if (state_dt == DT_BF16 && op_dt == DT_BF16) MUONH_MOM(bf16_t, bf16_t);
  else if (state_dt == DT_BF16 && op_dt == DT_F32) MUONH_MOM(bf16_t, float);
  else if (state_dt == DT_F32 && op_dt == DT_BF16) MUONH_MOM(float, bf16_t);
  else MUONH_MOM(float, float);
#undef MUONH_MOM
  return hipGetLastError();
}

hipError_t launch_hook_reduce(int mode, const HookMat* mats, const HookBlock* blocks, int nblocks,
                              const SlotTable& st, float eta, hipStream_t s) {
  if (nblocks <= 0) return hipSuccess;
  if (mode == kModeRB)
    hipLaunchKernelGGL((k_hook_reduce<kModeRB>), dim3(nblocks), dim3(kHookThreads), 0, s, mats, blocks, st, eta);
  else if (mode == kModeRel)
    hipLaunchKernelGGL((k_hook_reduce<kModeRel>), dim3(nblocks), dim3(kHookThreads), 0, s, mats, blocks, st, eta);
  else
    hipLaunchKernelGGL((k_hook_reduce<kModeHB>), dim3(nblocks), dim3(kHookThreads), 0, s, mats, blocks, st, eta);
  return hipGetLastError();
}

hipError_t launch_hook_write(int mode, const HookMat* mats, const HookBlock* blocks, int nblocks,
                             const SlotTable& st, float eta, float zero_rel_eps, float outward,
                             float inward, float rb_eps, float decay, Flags* flags, hipStream_t s) {
  if (nblocks <= 0) return hipSuccess;
#define MUONH_HW(MODE)                                                                                   \
  hipLaunchKernelGGL((k_hook_write<MODE>), dim3(nblocks), dim3(kHookThreads), 0, s, mats, blocks, st, eta, \
                     zero_rel_eps, outward, inward, rb_eps, decay, flags)
  if (mode == kModeRB) MUONH_HW(kModeRB);
  else if (mode == kModeNone) MUONH_HW(kModeNone);
  else if (mode == kModeRel) MUONH_HW(kModeRel);
  else MUONH_HW(kModeHB);
#undef MUONH_HW
  return hipGetLastError();
}

hipError_t launch_adam_moments(int g_dt, bool sums, const HookMat* mats, const HookBlock* blocks, int nblocks,
                               const SlotTable& st, const AdamArgs& a, hipStream_t s) {
  if (nblocks <= 0) return hipSuccess;
#define MUONH_AM(GT, S) \
  hipLaunchKernelGGL((k_adam_moments<GT, S>), dim3(nblocks), dim3(kHookThreads), 0, s, mats, blocks, st, a)
  if (g_dt == DT_BF16) {
    if (sums) MUONH_AM(bf16_t, true);
    else MUONH_AM(bf16_t, false);
  } else {
    if (sums) MUONH_AM(float, true);
    else MUONH_AM(float, false);
  }
#undef MUONH_AM
  return hipGetLastError();
}

hipError_t launch_adam_write(int mode, const HookMat* mats, const HookBlock* blocks, int nblocks, const SlotTable& st,
                             const AdamArgs& a, float eta, float zero_rel_eps, float outward, float inward,
                             float rb_eps, float decay, Flags* flags, hipStream_t s) {
  if (nblocks <= 0) return hipSuccess;
#define MUONH_AW(MODE)                                                                                    \
  hipLaunchKernelGGL((k_adam_write<MODE>), dim3(nblocks), dim3(kHookThreads), 0, s, mats, blocks, st, a, eta, \
                     zero_rel_eps, outward, inward, rb_eps, decay, flags)
  if (mode == kModeRB) MUONH_AW(kModeRB);
  else if (mode == kModeNone) MUONH_AW(kModeNone);
  else if (mode == kModeRel) MUONH_AW(kModeRel);
  else MUONH_AW(kModeHB);
#undef MUONH_AW
  return hipGetLastError();
}

hipError_t launch_sumsq(const HookMat* mats, const HookBlock* blocks, int nblocks, const SlotTable& st,
                        hipStream_t s) {
  if (nblocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_sumsq, dim3(nblocks), dim3(kHookThreads), 0, s, mats, blocks, st);
  return hipGetLastError();
}

hipError_t launch_finalize(const SlotTable& st, int slot0, int nslots, hipStream_t s) {
  if (nslots <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_finalize, dim3(nslots), dim3(256), 0, s, st, slot0);
  return hipGetLastError();
}

}  // namespace muonh
