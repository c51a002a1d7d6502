// Host-side planner of libmuonh (no HIP runtime calls).
//
// Units.  Full-matrix Newton-Schulz works on the wide side of each matrix
// (Muon explainer, code section: a tall matrix is transposed so that X X^T is
// the small Gram); here that is only a layout flag.  Hierarchical Muon
// ("Hierarchical Muon: Tiled Newton-Schulz Updates for Efficient Muon
// Optimization", core claim) cuts each matrix into T x T tiles from (0, 0);
// every tile becomes its own zero-padded T x T unit.
//
// Chunks.  Matrices are taken in order and packed into chunks whose
// workspace fits the limit (the memory-bounded chunking that page lists
// among the tiled scheme's implementation options); each chunk runs the whole
// step before the next one reuses the workspace.  When the whole set fits in
// one chunk it is cut into up to four runs instead (lanes): the caller runs
// them on as many streams, so that one lane's launches fill the gaps and
// drain tails of another's and its streaming passes (momentum, hook) overlap
// the other lanes' Newton-Schulz products.  Matrices never interact, so the
// results do not depend on the split.
#include "planner.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>

#include "muonh.h"

namespace muonh {

UnitBytes unit_bytes(int r, int s, int op_dt, int x32) {
  const int64_t es = esize(op_dt);
  const int64_t ld_s = pad_up(s, kPad), ld_r = pad_up(r, kPad);
  // GEMM operands hold whole 256-row tiles, and X^T a further 256 elements
  // (the column overrun of a transposed 256-wide tile on its last row): the
  // 256-tile main loop loads whole tiles without clamping; the rows past the
  // true sides only feed outputs that are never stored.
  const int64_t rows_s = pad_up(s, 256), rows_r = pad_up(r, 256);
  UnitBytes u;
  u.xt = align256((rows_s * ld_r + 256) * es);
  u.x32 = (x32 && op_dt == DT_BF16) ? align256(ld_s * ld_r * 4) : 0;
  u.a = align256(rows_r * ld_r * es);
  u.b = u.a;
  return u;
}

// 256-tiles (the ping-pong main loop) for bf16 units with r >= 1024 (>= 10
// upper tiles for G1 / G2, >= 16 tiles for G3 per unit), and for G3 already
// from r >= 512; smaller units keep 128-tiles, which fill the chip better.
// MUONH_GEMM_BIG=0 / 2 forces 128 / 256 tiles (bf16) for tuning runs;
// results do not depend on the choice beyond summation order.
bool tile256_enabled() {
  static int on = -1;
  if (on < 0) {
    const char* e = std::getenv("MUONH_TILE256");
    on = (e && *e) ? (std::atoi(e) != 0) : 1;
  }
  return on != 0;
}

int unit_gemm_cfg(int r, int op_dt, bool phase12) {
  // fp32 units with r <= 256 (a product of at most a few 128-tiles) run on
  // 64-tiles: four times the workgroups for the same latency-bound work
  if (op_dt != DT_BF16) return r <= 256 ? 2 : 0;
  static int mode = -1;
  if (mode < 0) {
    const char* e = std::getenv("MUONH_GEMM_BIG");
    mode = (e && *e) ? std::atoi(e) : 1;
  }
  if (mode == 0) return 0;
  if (mode == 2) return 1;
  return r >= (phase12 ? 1024 : 512) ? 1 : 0;
}

static int64_t jobs_per_iter(int r, int s, int op_dt) {
  const int B12 = gemm_tile_side(unit_gemm_cfg(r, op_dt, true));
  const int B3 = gemm_tile_side(unit_gemm_cfg(r, op_dt, false));
  const int64_t nr12 = (pad_up(r, kPad) + B12 - 1) / B12;
  const int64_t nr = (pad_up(r, kPad) + B3 - 1) / B3, ns = (pad_up(s, kPad) + B3 - 1) / B3;
  return 2 * (nr12 * (nr12 + 1) / 2) + nr * ns;  // symmetric G1, G2 + G3
}

// AdamH bytes per element: pass 1 reads g, m, v (and W for the hook's
// norms) and writes m, v; pass 2 reads W, m, v and writes W.
static double adam_bytes_per_elem(const Cfg& cfg) {
  const double gb = esize(cfg.state_dt);
  return (gb + 16 + (cfg.hook == kModeNone ? 0 : 4)) + 16;
}

static double ns_flops_true(int64_t h, int64_t w, int K) {
  const double r = (double)std::min(h, w), s = (double)std::max(h, w);
  return (double)K * (4.0 * r * r * s + 2.0 * r * r * r);
}

int make_plan(const int64_t* shapes, const Cfg& cfg, Plan& plan) {
  plan = Plan();
  const int n = cfg.n;
  plan.mats.resize(n);
  bool all_engine = true;    // every matrix on the GEMM engine (full NS, or tiles above the resident size)
  bool all_resident = true;  // every matrix on a resident-tile kernel
  for (int i = 0; i < n; ++i) {
    MatPlan& m = plan.mats[i];
    const int T = mat_tile(cfg, i);
    m.T = no_ns(cfg.kind) ? 0 : T;
    all_engine = all_engine && !resident_tile(cfg, m.T);
    all_resident = all_resident && resident_tile(cfg, m.T);
    m.H = shapes[2 * i];
    m.W = shapes[2 * i + 1];
    if (m.H < 1 || m.W < 1 || m.H > (int64_t)1 << 30 || m.W > (int64_t)1 << 30) return MUONH_EINVAL;
    if (m.H * m.W > ((int64_t)1 << 40)) return MUONH_EINVAL;
    m.ws_bytes = 0;
    const int64_t numel = m.H * m.W;
    if (no_ns(cfg.kind)) {
      m.r = (int)std::min(m.H, m.W);
      m.s = (int)std::max(m.H, m.W);
      m.trans = m.H > m.W;
      m.nunits = 0;
      m.ntr = m.ntc = 0;
      const double ob = cfg.state_dt == DT_F32 ? 4 : 2;
      if (cfg.kind == CALL_PROJ) plan.stream_bytes += (double)numel * (ob + (4 + ob) + (4 + ob + 4));
      else plan.stream_bytes += (double)numel * adam_bytes_per_elem(cfg);
      continue;
    }
    if (T > 0) {
      m.r = m.s = T;
      m.trans = 0;
      m.ntr = (int)((m.H + T - 1) / T);
      m.ntc = (int)((m.W + T - 1) / T);
      m.nunits = m.ntr * m.ntc;
      for (int a = 0; a < m.ntr; ++a)
        for (int b = 0; b < m.ntc; ++b) {
          const int64_t h = std::min<int64_t>(T, m.H - (int64_t)a * T);
          const int64_t w = std::min<int64_t>(T, m.W - (int64_t)b * T);
          plan.ns_flops += ns_flops_true(h, w, cfg.K);
        }
      if (resident_tile(cfg, T)) {
        plan.jobs_per_iter += m.nunits;  // one workgroup per tile runs every iteration
      } else {
        const UnitBytes ub = unit_bytes(T, T, cfg.op_dt, cfg.x32 || cfg.seed32);
        m.ws_bytes += (int64_t)m.nunits * ub.total();
        plan.jobs_per_iter += (int64_t)m.nunits * jobs_per_iter(T, T, cfg.op_dt);
      }
    } else {
      m.r = (int)std::min(m.H, m.W);
      m.s = (int)std::max(m.H, m.W);
      m.trans = m.H > m.W ? 1 : 0;
      m.nunits = 1;
      m.ntr = m.ntc = 1;
      // GEMM operand loads address a unit's X^T with 32-bit byte offsets.
      if ((pad_up(m.s, 256) * pad_up(m.r, kPad) + 256) * esize(cfg.op_dt) >= ((int64_t)1 << 32)) return MUONH_ENOTIMPL;
      const UnitBytes ub = unit_bytes(m.r, m.s, cfg.op_dt, cfg.x32 || cfg.seed32);
      m.ws_bytes += ub.total();
      plan.ns_flops += ns_flops_true(m.H, m.W, cfg.K);
      plan.jobs_per_iter += jobs_per_iter(m.r, m.s, cfg.op_dt);
    }
    if (cfg.kind == CALL_STEP) m.ws_bytes += align256(numel * esize(cfg.op_dt));  // O
    plan.units += m.nunits;
    const double sb = cfg.state_dt == DT_F32 ? 4 : 2;
    const double ob = esize(cfg.op_dt);
    // momentum 3 passes; hook pass 1 (none for Muon's own update; W only for
    // RelativeUpdate) and pass 2
    // hook pass 1: W and O (RelativeUpdate: W only); with resident tiles
    // the tile kernel reads W for the norms instead (4 bytes)
    const bool fused_mat = cfg.kind == CALL_STEP && cfg.hook != kModeNone && resident_tile(cfg, T);
    const double hook1 = cfg.hook == kModeNone ? 0 : (cfg.hook == kModeRel || fused_mat) ? 4 : 4 + ob;
    if (cfg.kind == CALL_STEP) plan.stream_bytes += (double)numel * (3 * sb + hook1 + (4 + ob + 4));
    else plan.stream_bytes += (double)numel * (sb + sb);  // NS: read input, write output
  }
  // chunks: the fewest runs of consecutive matrices whose workspace fits the
  // limit (greedy packing), then the same count re-cut at the smallest
  // per-chunk cap that still packs into it, so chunks come out about equal
  // (8B-shaped set, 16 GiB: four chunks of eight layers, not three of ten and
  // a last one of two), each launch as full as the others.
  const int64_t limit = (int64_t)cfg.ws_limit;
  int64_t biggest = 0;
  for (int i = 0; i < n; ++i) {
    if (plan.mats[i].ws_bytes > limit) return MUONH_ENOMEM;
    biggest = std::max(biggest, plan.mats[i].ws_bytes);
  }
  auto pack = [&](int64_t cap, bool emit) {
    int m0 = 0, count = 1;
    int64_t acc = 0;
    for (int i = 0; i < n; ++i) {
      const int64_t b = plan.mats[i].ws_bytes;
      if (acc + b > cap && i > m0) {
        if (emit) plan.chunks.push_back({m0, i, acc, 0});
        m0 = i;
        acc = 0;
        ++count;
      }
      acc += b;
    }
    if (emit) plan.chunks.push_back({m0, n, acc, 0});
    return count;
  };
  const int nchunks = pack(limit, false);
  int64_t lo = biggest, hi = limit;  // pack(hi) <= nchunks always holds
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo) / 2;
    if (pack(mid, false) <= nchunks) hi = mid;
    else lo = mid + 1;
  }
  pack(hi, true);
  for (auto& c : plan.chunks) plan.ws_bytes = std::max(plan.ws_bytes, c.ws_bytes);
  // Automatic choice: two lanes, except (one lane) for Newton-Schulz on the
  // GEMM engine (full matrices, or tiles above the resident size) with a long
  // iteration, where launch gaps are negligible and the lanes' large products
  // only contend for the caches (measured slower: 1.2B set full), and when
  // every matrix runs on a resident-tile kernel: one launch per lane has no
  // gaps to fill, and two concurrent tile launches each leave a partial last
  // round (GPT-2-small set at T = 64 / 128 / 256: one lane 1% / 3% / 2%
  // faster).
  const double iter_flops = plan.ns_flops / std::max(cfg.K, 1);
  const bool one = all_resident || (all_engine && iter_flops > kAutoLaneIterFlops);
  const int want = cfg.lanes > 0 ? cfg.lanes : (one ? 1 : 2);
  const int L = std::min(want, n);
  if (plan.chunks.size() == 1 && L >= 2 && !no_ns(cfg.kind)) {
    // Lanes: cut the set into L runs of matrices whose Newton-Schulz work is
    // as equal as the order allows (each cut at the prefix sum nearest to
    // l/L of the total, every run non-empty).  The runs own disjoint
    // workspace regions (the same total as one chunk) and run concurrently.
    std::vector<double> f(n), pre(n + 1, 0.0);
    for (int i = 0; i < n; ++i) {
      const MatPlan& m = plan.mats[i];
      f[i] = m.nunits > 1 ? (double)m.nunits * ns_flops_true(m.r, m.s, cfg.K) : ns_flops_true(m.H, m.W, cfg.K);
      pre[i + 1] = pre[i] + f[i];
    }
    std::vector<int> cut(L + 1, 0);
    cut[L] = n;
    for (int l = 1; l < L; ++l) {
      const double target = pre[n] * l / L;
      int best = cut[l - 1] + 1;
      for (int i = best; i <= n - (L - l); ++i)
        if (std::fabs(pre[i] - target) < std::fabs(pre[best] - target)) best = i;
      cut[l] = best;
    }
    plan.chunks.clear();
    int64_t off = 0;
    for (int l = 0; l < L; ++l) {
      int64_t bytes = 0;
      for (int i = cut[l]; i < cut[l + 1]; ++i) bytes += plan.mats[i].ws_bytes;
      plan.chunks.push_back({cut[l], cut[l + 1], bytes, off});
      off += bytes;
    }
    plan.ws_bytes = off;
    plan.lanes = L;
  }
  return MUONH_OK;
}

void fill_chunk(const Plan& plan, int c, const Cfg& cfg, const CallPtrs& p, char* ws, ChunkTables& t) {
  t = ChunkTables();
  const ChunkPlan& ch = plan.chunks[c];
  const int nm = ch.m1 - ch.m0;
  const int es_op = esize(cfg.op_dt);

  // --- units and workspace carve
  int64_t off = ch.ws_off;
  auto carve = [&](int64_t bytes) -> char* {
    char* q = ws + off;
    off += bytes;
    return q;
  };
  std::vector<int> unit0(nm);
  std::vector<char*> obuf(nm, nullptr);
  for (int mi = 0; mi < nm; ++mi) {
    const MatPlan& m = plan.mats[ch.m0 + mi];
    unit0[mi] = (int)t.units.size();
    if (no_ns(cfg.kind)) continue;
    if (resident_tile(cfg, m.T)) {
      if (cfg.kind == CALL_STEP) obuf[mi] = carve(align256(m.H * m.W * es_op));
      continue;
    }
    const UnitBytes ub = unit_bytes(m.r, m.s, cfg.op_dt, cfg.x32 || cfg.seed32);
    for (int k = 0; k < m.nunits; ++k) {
      NsUnit u{};
      u.r = m.r;
      u.s = m.s;
      u.ld_s = (int32_t)pad_up(m.s, kPad);
      u.ld_r = (int32_t)pad_up(m.r, kPad);
      u.xt[0] = carve(ub.xt);
      u.xt[1] = carve(ub.xt);
      u.x32 = ub.x32 ? reinterpret_cast<float*>(carve(ub.x32)) : nullptr;
      u.a = carve(ub.a);
      u.b = carve(ub.b);
      t.units.push_back(u);
    }
    if (cfg.kind == CALL_STEP) obuf[mi] = carve(align256(m.H * m.W * es_op));
  }
  const int nunits = (int)t.units.size();
  auto resident = [&](const MatPlan& m) { return !no_ns(cfg.kind) && resident_tile(cfg, m.T); };
  // A step's hook norms (<W, O>, ||W||^2) are summed where O is stored for
  // matrices run as resident tiles: the tile kernel reads W at little cost,
  // while in the GEMM engine's last epilogue the extra read costs more than
  // the separate norm pass it would replace.
  auto fused = [&](const MatPlan& m) { return cfg.kind == CALL_STEP && cfg.hook != kModeNone && resident(m); };

  // --- slots: [unit norms][matrix O norms][matrix hook sums]; the
  // resident-tile kernel forms its tile norms itself, so it has no unit slots.
  const int s_norm0 = 0, s_onorm0 = nunits, s_hook0 = nunits + nm;
  const int nslots = nunits + 2 * nm;
  t.nparts.assign(nslots, 0);

  // --- resident tiles: one job per tile, momentum fused; one launch per
  // distinct tile side, in increasing order
  {
    std::vector<int> sides;
    for (int mi = 0; mi < nm; ++mi) {
      const MatPlan& m = plan.mats[ch.m0 + mi];
      if (resident(m) && std::find(sides.begin(), sides.end(), m.T) == sides.end()) sides.push_back(m.T);
    }
    std::sort(sides.begin(), sides.end());
    const double sb = esize(cfg.state_dt);
    for (const int T : sides) {
      TileGroup grp{T, (int)t.tile_jobs.size(), 0, 0.0, 0.0};
      for (int mi = 0; mi < nm; ++mi) {
        const int gi = ch.m0 + mi;
        const MatPlan& m = plan.mats[gi];
        if (!resident(m) || m.T != T) continue;
        TileMat tm{};
        tm.g = cfg.kind == CALL_STEP ? p.grads[gi] : nullptr;
        tm.m = cfg.kind == CALL_STEP ? p.moms[gi] : const_cast<void*>(p.grads[gi]);
        tm.out = cfg.kind == CALL_STEP ? (void*)obuf[mi] : p.outs[gi];
        tm.H = m.H;
        tm.W = m.W;
        tm.out_dtype = cfg.kind == CALL_STEP ? cfg.op_dt : cfg.state_dt;
        tm.onorm_slot = s_onorm0 + mi;
        tm.hook_slot = s_hook0 + mi;
        tm.w = fused(m) ? static_cast<const float*>(p.params[gi]) : nullptr;
        // 8-element (16 / 32-byte) chunks need 8-aligned rows and tile origins
        // and 16-byte aligned buffers.
        auto a16 = [](const void* q) { return ((uintptr_t)q & 15) == 0; };
        tm.vec = (m.W % 8 == 0 && T % 8 == 0 && a16(tm.g) && a16(tm.m) && a16(tm.out) && a16(tm.w)) ? 1 : 0;
        const int idx = (int)t.tile_mats.size();
        t.tile_mats.push_back(tm);
        for (int a = 0; a < m.ntr; ++a)
          for (int b = 0; b < m.ntc; ++b) {
            t.tile_jobs.push_back({idx, a, b, a * m.ntc + b});
            const int64_t h = std::min<int64_t>(T, m.H - (int64_t)a * T);
            const int64_t w = std::min<int64_t>(T, m.W - (int64_t)b * T);
            grp.flops += ns_flops_true(h, w, cfg.K);
          }
        t.nparts[s_onorm0 + mi] = m.nunits;
        const double numel = (double)m.H * m.W;
        // read G and M, write M and O; the hook's W read where it is fused
        grp.bytes += cfg.kind == CALL_STEP ? numel * (3 * sb + es_op + (fused(m) ? 4 : 0)) : numel * 2 * sb;
      }
      grp.njobs = (int)t.tile_jobs.size() - grp.job0;
      t.flops_tile += grp.flops;
      t.bytes_tile += grp.bytes;
      t.tile_groups.push_back(grp);
    }
  }

  // --- output placement, O-norm partial numbering, GEMM jobs, flops
  for (int mi = 0; mi < nm; ++mi) {
    const int gi = ch.m0 + mi;
    const MatPlan& m = plan.mats[gi];
    if (no_ns(cfg.kind) || resident(m)) continue;
    const int T = m.T;
    void* out = cfg.kind == CALL_STEP ? (void*)obuf[mi] : p.outs[gi];
    const int out_dt = cfg.kind == CALL_STEP ? cfg.op_dt : cfg.state_dt;
    const int oes = esize(out_dt);
    int part = 0;
    for (int k = 0; k < m.nunits; ++k) {
      NsUnit& u = t.units[unit0[mi] + k];
      u.norm_slot = s_norm0 + unit0[mi] + k;
      u.onorm_slot = s_onorm0 + mi;
      u.onorm_part0 = part;
      u.o_dtype = out_dt;
      u.o_ld = m.W;
      int64_t h, w;
      if (T > 0) {
        const int a = k / m.ntc, b = k % m.ntc;
        h = std::min<int64_t>(T, m.H - (int64_t)a * T);
        w = std::min<int64_t>(T, m.W - (int64_t)b * T);
        u.o_trans = 0;
        u.o_rows = (int32_t)h;
        u.o_cols = (int32_t)w;
        u.o_ptr = static_cast<char*>(out) + ((int64_t)a * T * m.W + (int64_t)b * T) * oes;

      } else {
        h = m.H;
        w = m.W;
        u.o_trans = m.trans;
        u.o_rows = m.r;
        u.o_cols = m.s;
        u.o_ptr = out;

      }
      const int gc12 = unit_gemm_cfg(u.r, cfg.op_dt, true), gc3 = unit_gemm_cfg(u.r, cfg.op_dt, false);
      const int B12 = gemm_tile_side(gc12), B3 = gemm_tile_side(gc3);
      const int n12 = (u.ld_r + B12 - 1) / B12;
      const int g3r = (u.ld_r + B3 - 1) / B3, g3c = (u.ld_s + B3 - 1) / B3;
      u.g3_cols = g3c;
      part += g3r * g3c;
      const int uid = unit0[mi] + k;
      // A and B are symmetric: only tiles on or above the diagonal, the
      // epilogue mirrors the off-diagonal ones.
      for (int tm = 0; tm < n12; ++tm)
        for (int tn = tm; tn < n12; ++tn) t.g12_jobs[gc12].push_back({uid, tm, tn, u.ld_r / 64});
      // G3 jobs in column order while a column has at most 8 tiles; taller
      // units go in blocks of 4 tile rows x 8 tile columns, so the 32
      // workgroups one XCD runs together (its run of the job list) share
      // 4 panels of B and 8 of X^T, against 16 + 2 in column order (r = 4096:
      // 3% less G3 time; at 8 rows both orders touch 12 panels and column
      // order measured no slower).
      {
        const int br = g3r <= 8 ? g3r : 4, bc = 32 / br;
        for (int tn0 = 0; tn0 < g3c; tn0 += bc)
          for (int tm0 = 0; tm0 < g3r; tm0 += br)
            for (int tn = tn0; tn < std::min(tn0 + bc, g3c); ++tn)
              for (int tm = tm0; tm < std::min(tm0 + br, g3r); ++tm)
                t.g3_jobs[gc3].push_back({uid, tm, tn, u.ld_r / 64});
      }
      const double r = (double)std::min(h, w), s = (double)std::max(h, w);
      t.flops_g1[gc12] += 2.0 * r * r * s;
      t.flops_g2[gc12] += 2.0 * r * r * r;
      t.flops_g3[gc3] += 2.0 * r * r * s;
    }
    t.nparts[s_onorm0 + mi] = part;
  }
  // Within the run of the G1 / G2 job list that one XCD takes (the kernels'
  // block -> job map gives XCD x the x-th of 8 near-equal contiguous runs),
  // units with deeper Grams (G1 contracts over s) go first, so each run ends
  // on its shortest jobs; a unit's own jobs keep their order.  GPT-2-small
  // set (fc and proj Grams 4 times as deep as attn-out's): G1 7% faster; the
  // 8B-shaped set (a run is one layer, gate / up / down 3.5 times as deep):
  // G1 0.7% faster.  G3 keeps the unit order: its k / v jobs moved to the
  // end of each layer measured 0.6% slower.
  for (int g = 0; g < kGemmCfgs; ++g) {
    std::vector<GemmJob>& v = t.g12_jobs[g];
    const int nj = (int)v.size(), q = nj / 8, rem = nj % 8;
    for (int x = 0, b = 0; x < 8; ++x) {
      const int e = b + q + (x < rem ? 1 : 0);
      std::stable_sort(v.begin() + b, v.begin() + e, [&](const GemmJob& l, const GemmJob& r) {
        return t.units[l.unit].ld_s > t.units[r.unit].ld_s;
      });
      b = e;
    }
  }

  // --- momentum / prep blocks
  if (!no_ns(cfg.kind)) {
    for (int mi = 0; mi < nm; ++mi) {
      const int gi = ch.m0 + mi;
      const MatPlan& m = plan.mats[gi];
      if (resident(m)) continue;
      const int T = m.T;
      MomMat mm{};
      mm.g = p.grads[gi];
      mm.m = cfg.kind == CALL_STEP ? p.moms[gi] : nullptr;
      mm.H = m.H;
      mm.W = m.W;
      mm.trans = T > 0 ? 0 : m.trans;
      mm.tile_T = T;
      mm.unit0 = unit0[mi];
      mm.ntc = m.ntc;
      mm.write_x = 1;
      mm.write_x32 = cfg.seed32;
      int64_t rows_p, cols_p;
      if (T > 0) {
        rows_p = (int64_t)m.ntr * T;
        cols_p = (int64_t)m.ntc * T;
      } else {
        rows_p = pad_up(m.H, 64);
        cols_p = pad_up(m.W, 64);
      }
      const int nbr = (int)(rows_p / 64), nbc = (int)(cols_p / 64);
      mm.nbc = nbc;
      const int mat_idx = (int)t.mom_mats.size();
      t.mom_mats.push_back(mm);
      for (int br = 0; br < nbr; ++br)
        for (int bc = 0; bc < nbc; ++bc) {
          MomBlock b{};
          b.mat = mat_idx;
          b.br = br;
          b.bc = bc;
          if (T > 0) {
            const int tr = (int)((int64_t)br * 64 / T), tc = (int)((int64_t)bc * 64 / T);
            const int per = T / 64;
            b.slot = s_norm0 + unit0[mi] + tr * m.ntc + tc;
            b.part = ((br * 64 % T) / 64) * per + (bc * 64 % T) / 64;
          } else {
            b.slot = s_norm0 + unit0[mi];
            b.part = br * nbc + bc;
          }
          t.mom_blocks.push_back(b);
        }
      const int per_slot = T > 0 ? (T / 64) * (T / 64) : nbr * nbc;
      for (int k = 0; k < m.nunits; ++k) t.nparts[s_norm0 + unit0[mi] + k] = per_slot;
      const double sb = esize(cfg.state_dt);
      t.bytes_mom += (double)m.H * m.W * (cfg.kind == CALL_STEP ? 3 * sb : sb);
    }
  }

  // --- hook / projection blocks
  if (cfg.kind != CALL_NS) {
    for (int mi = 0; mi < nm; ++mi) {
      const int gi = ch.m0 + mi;
      const MatPlan& m = plan.mats[gi];
      HookMat hm{};
      hm.w = static_cast<float*>(p.params[gi]);
      hm.numel = m.H * m.W;
      hm.nblocks = (int)((hm.numel + kHookBlockElems - 1) / kHookBlockElems);
      hm.slot = s_hook0 + mi;
      hm.rho = p.rho ? p.rho[gi] : 1.0f;
      hm.oscale = cfg.hook == kModeHB ? (cfg.hb_radius ? hm.rho : 1.0f)
                                      : (float)std::sqrt(std::max(1.0, (double)m.H / (double)m.W));
      if (cfg.kind == CALL_ADAM) {
        // Adam's direction has no shape scale (that is Muon's)
        if (cfg.hook != kModeHB) hm.oscale = 1.0f;
        hm.o = p.grads[gi];
        hm.o_dtype = cfg.state_dt;
        hm.am = static_cast<float*>(p.moms[gi]);
        hm.av = static_cast<float*>(p.vs[gi]);
        hm.onorm_slot = s_onorm0 + mi;
        t.nparts[s_onorm0 + mi] = hm.nblocks;
        t.nparts[s_hook0 + mi] = hm.nblocks;
        const int idx = (int)t.hook_mats.size();
        t.hook_mats.push_back(hm);
        for (int b = 0; b < hm.nblocks; ++b) t.hook_blocks.push_back({idx, b});
        const double gb = esize(cfg.state_dt);
        t.bytes_hook1 += (double)hm.numel * (gb + 16 + (cfg.hook == kModeNone ? 0 : 4));
        t.bytes_hook2 += (double)hm.numel * 16;
        continue;
      }
      if (cfg.kind == CALL_STEP) {
        hm.o = obuf[mi];
        hm.o_dtype = cfg.op_dt;
        hm.onorm_slot = s_onorm0 + mi;
      } else {
        const void* U = p.grads ? p.grads[gi] : nullptr;
        hm.o = U;
        hm.o_dtype = cfg.state_dt;
        hm.onorm_slot = U ? s_onorm0 + mi : -1;
        if (U) t.nparts[s_onorm0 + mi] = hm.nblocks;
      }
      // fused: one (0, ||W||^2) partial per O-norm partial (per tile)
      hm.fused = fused(m) ? 1 : 0;
      t.nparts[s_hook0 + mi] = hm.fused ? t.nparts[s_onorm0 + mi] : hm.nblocks;
      const int idx = (int)t.hook_mats.size();
      t.hook_mats.push_back(hm);
      for (int b = 0; b < hm.nblocks; ++b) {
        t.hook_blocks.push_back({idx, b});
        if (!hm.fused) t.hook1_blocks.push_back({idx, b});
      }
      const double ob = hm.o ? esize(hm.o_dtype) : 0;
      if (hm.fused) {
        // no pass 1
      } else if (cfg.hook == kModeRel) {
        t.bytes_hook1 += (double)hm.numel * 4;  // ||W||^2 only
      } else if (cfg.hook != kModeNone) {
        t.bytes_hook1 += (double)hm.numel * (4 + ob);
      }
      t.bytes_hook2 += (double)hm.numel * (4 + ob + 4);
      if (cfg.kind == CALL_PROJ && hm.o) t.bytes_sumsq += (double)hm.numel * ob;
    }
  }

  // --- partial bases
  t.part_base.assign(nslots, 0);
  int64_t acc = 0;
  for (int s = 0; s < nslots; ++s) {
    t.part_base[s] = acc;
    acc += t.nparts[s];
  }
  t.parts_total = acc;
}

}  // namespace muonh
