// libmuonh C ABI: validation, workspace, cached descriptor tables, launch
// sequencing and measurement hooks.  The per-step sequence for one chunk of
// matrices is
//   k_momentum_prep                      (momentum, ||M||^2, X0 layouts)
//   K x { G1 gram, G2 poly, G3 update }  (Newton-Schulz, grouped MFMA GEMMs)
//   k_hook_reduce, k_hook_write          (Hyperball or RadialBrake)
// all queued on the caller's stream with no host synchronization.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <list>
#include <mutex>
#include <string>
#include <vector>

#include "muonh.h"
#include "desc.h"
#include "planner.h"

// Device memory the library holds without allocating it: the flag counters of
// every entry point, and the scratch of muonh_step_noalloc (its workspace,
// descriptor tables and reduction partials), one copy per GPU for the life of
// the process.  Host code never passes these names to a kernel: it takes each
// GPU's addresses from hipGetSymbolAddress (device_symbols below).
constexpr size_t kNoAllocScratchBytes = MUONH_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];
static __device__ __align__(256) muonh::Flags g_flags;

namespace muonh {

// launchers (kernels_*.hip)
hipError_t launch_momentum_prep(int state_dt, int op_dt, const MomMat* mats, const MomBlock* blocks,
                                int nblocks, const NsUnit* units, const SlotTable& st, float beta,
                                float gcoef, int nesterov, hipStream_t s);
hipError_t launch_hook_reduce(int mode, const HookMat* mats, const HookBlock* blocks, int nblocks,
                              const SlotTable& st, float eta, hipStream_t s);
hipError_t launch_hook_write(int mode, const HookMat* mats, const HookBlock* blocks, int nblocks,
                             const SlotTable& st, float eta, float zero_rel_eps, float outward,
                             float inward, float rb_eps, float decay, Flags* flags, hipStream_t s);
hipError_t launch_adam_moments(int g_dt, bool sums, const HookMat* mats, const HookBlock* blocks, int nblocks,
                               const SlotTable& st, const AdamArgs& a, hipStream_t s);
hipError_t launch_adam_write(int mode, const HookMat* mats, const HookBlock* blocks, int nblocks, const SlotTable& st,
                             const AdamArgs& a, float eta, float zero_rel_eps, float outward, float inward,
                             float rb_eps, float decay, Flags* flags, hipStream_t s);
hipError_t launch_sumsq(const HookMat* mats, const HookBlock* blocks, int nblocks, const SlotTable& st,
                        hipStream_t s);
hipError_t launch_finalize(const SlotTable& st, int slot0, int nslots, hipStream_t s);
hipError_t launch_ns_gemm(int op_dt, int out_dt, int phase, int cfg, const NsUnit* units, const GemmJob* jobs,
                          int njobs, float a, float b, float c, float eps, int first, int last, int cur,
                          int no_mma, int master32, int seed32, const SlotTable& st, hipStream_t s);
hipError_t launch_tile_ns(int state_dt, int op_dt, const TileMat* mats, const TileJob* jobs, int njobs,
                          const TileArgs& args, hipStream_t s);

namespace {

constexpr int kMaxK = 64;
static_assert(kMaxK == kTileMaxK, "iteration tables");

// ------------------------------------------------------------------ state
struct DevTables {  // one chunk's tables on the device
  char* mem = nullptr;
  bool mem_async = false;   // mem came from the stream-ordered allocator
  NsUnit* units = nullptr;
  GemmJob* g12[kGemmCfgs] = {};
  GemmJob* g3[kGemmCfgs] = {};
  MomMat* mom_mats = nullptr;
  MomBlock* mom_blocks = nullptr;
  HookMat* hook_mats = nullptr;
  HookBlock* hook_blocks = nullptr;
  HookBlock* hook1_blocks = nullptr;  // pass-1 blocks (matrices without fused norms)
  int n_hook1 = 0;
  TileMat* tile_mats = nullptr;
  TileJob* tile_jobs = nullptr;
  int n_tile = 0;
  std::vector<TileGroup> tile_groups;  // host copy: launch parameters
  double flops_tile = 0, bytes_tile = 0;
  int32_t* nparts = nullptr;
  int64_t* part_base = nullptr;
  int n_g12[kGemmCfgs] = {}, n_g3[kGemmCfgs] = {};
  int n_mom = 0, n_hook = 0;
  int64_t parts_total = 0;
  int nslots = 0;
  int nunits = 0, nmats = 0;  // slot ranges: [0,nunits) norms, then nmats O norms, then nmats hook sums
  int64_t part_off = 0;       // lanes: this chunk's first partial / slot in the shared arrays
  int slot_off = 0;
  double flops_g1[kGemmCfgs] = {}, flops_g2[kGemmCfgs] = {}, flops_g3[kGemmCfgs] = {};
  double bytes_mom = 0, bytes_hook1 = 0, bytes_hook2 = 0, bytes_sumsq = 0;
};

struct CachedPlan {
  std::vector<uint64_t> key;
  std::vector<DevTables> chunks;
  int64_t max_parts = 0;  // partials / slots the chunks need (sum over concurrent lanes)
  int max_slots = 0;
  int lanes = 1;
};

struct ProfRec {
  int cls;
  hipEvent_t e0, e1;
  double flops, bytes;
};

// Pinned host staging for descriptor-table uploads.  A buffer is reusable
// once the copy out of it has completed (its event); buffers are freed only
// by muonh_release, so a cache miss never frees host memory the device may
// still be reading.
struct Staging {
  char* p = nullptr;
  size_t cap = 0;
  hipEvent_t done = nullptr;
};

struct State {
  std::mutex mu;
  int device = -1;
  char* ws = nullptr;          // data workspace
  int64_t ws_bytes = 0;
  double* partials = nullptr;  // meta
  int64_t partials_cap = 0;
  double* sums = nullptr;
  int slots_cap = 0;
  // Meta buffers replaced by larger ones: kept until muonh_release, so that a
  // captured graph holding their addresses never writes freed memory.
  std::vector<void*> retired;
  std::vector<Staging> staging;
  std::vector<char> noalloc_blob;  // host copy of muonh_step_noalloc's last tables
  std::list<CachedPlan> plans;  // most recent first
  hipStream_t side[kMaxLanes] = {};  // lanes 1.. (created on first use; [0] unused)
  hipEvent_t ev_gate[kMaxLanes] = {}, ev_join[kMaxLanes] = {};
  bool profiling = false;
  std::vector<ProfRec> prof;
};

State& S() {
  static State s;
  return s;
}

const char* kClassNames[] = {"momentum_prep", "ns_gram_G1", "ns_poly_G2",       "ns_update_G3",
                             "hook_reduce",   "hook_write", "sumsq",            "finalize",
                             "ns_tile_resident", "adam_moments", "adam_write", "ns_tile_fused"};
enum { PC_MOM = 0, PC_G1, PC_G2, PC_G3, PC_HR, PC_HW, PC_SQ, PC_FIN, PC_TILE, PC_AM, PC_AW, PC_T256, PC_N };

// ------------------------------------------------------------------ helpers
// Frees a plan's device tables.  With a stream, stream-ordered allocations
// are released after the work already queued on it (no host wait); without
// one the device is synchronized first.
void free_plan(CachedPlan& p, hipStream_t s = nullptr, bool ordered = false) {
  for (auto& c : p.chunks) {
    if (!c.mem) continue;
    if (c.mem_async) {
      (void)hipFreeAsync(c.mem, ordered ? s : nullptr);
      if (!ordered) (void)hipStreamSynchronize(nullptr);
    } else {
      (void)hipFree(c.mem);
    }
    c.mem = nullptr;
  }
  p.chunks.clear();
}

// Drops every cached plan (workspace growth, muonh_release): waits for the
// device first, since queued work on any stream may still read the tables.
void clear_plans(State& st) {
  if (st.plans.empty()) return;
  (void)hipDeviceSynchronize();
  for (auto& p : st.plans) free_plan(p);
  st.plans.clear();
}

// Plan cache capacity (call signatures); least recently used out first.
constexpr size_t kPlanCacheSize = 32;

// Grows the reduction buffers.  A larger buffer is allocated before the old
// one is given up, so a failed allocation leaves the library as it was; the
// old buffer is retired, not freed (see State::retired).
int ensure_meta(State& st, int64_t parts, int slots) {
  if (parts > st.partials_cap) {
    const int64_t cap = std::max<int64_t>(parts, std::max<int64_t>(4096, 2 * st.partials_cap));
    double* p = nullptr;
    if (hipMalloc(&p, cap * 2 * sizeof(double)) != hipSuccess) return MUONH_ENOMEM;
    if (st.partials) st.retired.push_back(st.partials);
    st.partials = p;
    st.partials_cap = cap;
  }
  if (slots > st.slots_cap) {
    const int cap = std::max(slots, std::max(1024, 2 * st.slots_cap));
    double* p = nullptr;
    if (hipMalloc(&p, (size_t)cap * 2 * sizeof(double)) != hipSuccess) return MUONH_ENOMEM;
    if (st.sums) st.retired.push_back(st.sums);
    st.sums = p;
    st.slots_cap = cap;
  }
  return MUONH_OK;
}

int ensure_ws(State& st, int64_t bytes) {
  if (bytes <= st.ws_bytes) return MUONH_OK;
  // Growing invalidates every cached table (they hold workspace addresses);
  // hipFree waits for in-flight work that may still use the old buffer.
  clear_plans(st);
  if (st.ws) (void)hipFree(st.ws);
  st.ws = nullptr;
  st.ws_bytes = 0;
  if (hipMalloc(&st.ws, bytes) != hipSuccess) return MUONH_ENOMEM;
  st.ws_bytes = bytes;
  return MUONH_OK;
}

bool finite_f(float v) { return std::isfinite(v); }

struct Resolved {
  muonh_opts o;
  float coeffs[3 * kMaxK];
};

int resolve(const muonh_opts* in, int K, Resolved& r) {
  muonh_default_opts(&r.o);
  if (in) r.o = *in;
  const muonh_opts& o = r.o;
  if (o.param_dtype != MUONH_F32) return MUONH_EINVAL;  // fp32 master weights only
  if (o.deterministic != 0 && o.deterministic != 1) return MUONH_EINVAL;
  if (o.state_dtype != MUONH_BF16 && o.state_dtype != MUONH_F32) return MUONH_EINVAL;
  if (o.ns_dtype != MUONH_BF16 && o.ns_dtype != MUONH_F32) return MUONH_EINVAL;
  if (o.ns_precision != MUONH_NS_X32 && o.ns_precision != MUONH_NS_FOLD && o.ns_precision != MUONH_NS_H16)
    return MUONH_EINVAL;
  if (o.hyperball_step != MUONH_HB_STEP_UNIT && o.hyperball_step != MUONH_HB_STEP_RADIUS) return MUONH_EINVAL;
  if (o.hook != MUONH_HOOK_HYPERBALL && o.hook != MUONH_HOOK_RADIAL_BRAKE && o.hook != MUONH_HOOK_NONE &&
      o.hook != MUONH_HOOK_RELATIVE)
    return MUONH_EINVAL;
  if ((o.momentum_ema != 0 && o.momentum_ema != 1) || (o.nesterov != 0 && o.nesterov != 1)) return MUONH_EINVAL;
  if (!finite_f(o.weight_decay) || o.weight_decay < 0.f) return MUONH_EINVAL;
  if (o.lanes < 0 || o.lanes > kMaxLanes) return MUONH_EINVAL;
  if (!finite_f(o.ns_eps) || o.ns_eps < 0.f) return MUONH_EINVAL;
  if (!finite_f(o.zero_rel_eps) || o.zero_rel_eps < 0.f) return MUONH_EINVAL;
  if (!finite_f(o.rb_eps) || o.rb_eps < 0.f) return MUONH_EINVAL;
  // RadialBrake factors may damp but never amplify a radial change.
  if (!(o.outward >= 0.f && o.outward <= 1.f) || !(o.inward >= 0.f && o.inward <= 1.f)) return MUONH_EINVAL;
  for (int k = 0; k < K; ++k) {
    for (int j = 0; j < 3; ++j) {
      const float v = o.coeffs ? o.coeffs[3 * k + j] : (j == 0 ? 3.4445f : j == 1 ? -4.7750f : 2.0315f);
      if (!finite_f(v)) return MUONH_EINVAL;
      r.coeffs[3 * k + j] = v;
    }
  }
  return MUONH_OK;
}

int check_tile(int tile_T) {
  if (tile_T < 0) return MUONH_EINVAL;
  if (tile_T == 0) return MUONH_OK;
  if (tile_T > 8192) return MUONH_EINVAL;
  if (tile_T <= kTileResidentMax) return MUONH_OK;  // resident-tile kernel
  if (tile_T % 64 == 0) return MUONH_OK;             // GEMM engine
  return MUONH_EINVAL;
}

int check_tile_sizes(const int* sizes, int n) {
  if (!sizes) return MUONH_OK;
  for (int i = 0; i < n; ++i)
    if (check_tile(sizes[i]) != MUONH_OK) return MUONH_EINVAL;
  return MUONH_OK;
}

// 3/4 of the HBM free at the first call (fixed afterwards, so that chunking
// does not change as the library's own workspace grows).
size_t default_limit() {
  static size_t lim = 0;
  if (lim == 0) {
    size_t fr = 0, tot = 0;
    lim = hipMemGetInfo(&fr, &tot) == hipSuccess ? fr / 4 * 3 : (size_t)8 << 30;
  }
  return lim;
}

Cfg make_cfg(int kind, int n, int K, int tile_T, const Resolved& r, size_t limit) {
  Cfg c{};
  c.kind = kind;
  c.n = n;
  c.K = K;
  c.tile_T = tile_T;
  c.state_dt = r.o.state_dtype == MUONH_F32 ? DT_F32 : DT_BF16;
  c.op_dt = r.o.ns_dtype == MUONH_F32 ? DT_F32 : DT_BF16;
  c.x32 = (c.op_dt == DT_BF16 && r.o.ns_precision == MUONH_NS_X32) ? 1 : 0;
  c.h16 = (c.op_dt == DT_BF16 && r.o.ns_precision == MUONH_NS_H16) ? 1 : 0;
  // bf16 operands, NS input not a bf16 value: fp32 state, or the Nesterov blend
  c.seed32 = (c.op_dt == DT_BF16 && (c.state_dt == DT_F32 || (kind == CALL_STEP && r.o.nesterov))) ? 1 : 0;
  c.hook = r.o.hook == MUONH_HOOK_RADIAL_BRAKE ? kModeRB
           : r.o.hook == MUONH_HOOK_NONE        ? kModeNone
           : r.o.hook == MUONH_HOOK_RELATIVE    ? kModeRel
                                                : kModeHB;
  if (kind == CALL_PROJ) c.hook = kModeHB;  // frob_project is the Hyperball projection
  c.hb_radius = r.o.hyperball_step == MUONH_HB_STEP_RADIUS ? 1 : 0;
  c.ws_limit = limit;
  c.lanes = r.o.lanes;
  c.tile_sizes = no_ns(kind) ? nullptr : r.o.tile_sizes;
  return c;
}

template <typename T>
void put(std::vector<char>& blob, const std::vector<T>& v, size_t& off) {
  off = (blob.size() + 255) / 256 * 256;
  blob.resize(off + v.size() * sizeof(T));
  if (!v.empty()) memcpy(blob.data() + off, v.data(), v.size() * sizeof(T));
}

// Byte offsets of one chunk's tables inside its serialized blob.
struct BlobOffsets {
  size_t units, g12[kGemmCfgs], g3[kGemmCfgs], mm, mb, hm, hb, hb1, tm, tj, np, pb;
};

// Appends chunk t's tables to blob (each array 256-byte aligned) and records
// where each one starts.
void serialize_chunk(const ChunkTables& t, std::vector<char>& blob, BlobOffsets& o) {
  put(blob, t.units, o.units);
  for (int g = 0; g < kGemmCfgs; ++g) {
    put(blob, t.g12_jobs[g], o.g12[g]);
    put(blob, t.g3_jobs[g], o.g3[g]);
  }
  put(blob, t.mom_mats, o.mm);
  put(blob, t.mom_blocks, o.mb);
  put(blob, t.hook_mats, o.hm);
  put(blob, t.hook_blocks, o.hb);
  put(blob, t.hook1_blocks, o.hb1);
  put(blob, t.tile_mats, o.tm);
  put(blob, t.tile_jobs, o.tj);
  put(blob, t.nparts, o.np);
  put(blob, t.part_base, o.pb);
  blob.resize((blob.size() + 255) / 256 * 256 + 256);
}

// Points d at the device copy of a blob (base = device address of the
// blob's first byte) and copies the host-side launch parameters.
void bind_chunk(const ChunkTables& t, const BlobOffsets& o, char* base, DevTables& d) {
  d.mem = base;
  const size_t o_units = o.units, o_mm = o.mm, o_mb = o.mb, o_hm = o.hm, o_hb = o.hb, o_hb1 = o.hb1, o_tm = o.tm,
               o_tj = o.tj, o_np = o.np, o_pb = o.pb;
  const size_t* o_g12 = o.g12;
  const size_t* o_g3 = o.g3;
  d.units = reinterpret_cast<NsUnit*>(d.mem + o_units);
  for (int g = 0; g < kGemmCfgs; ++g) {
    d.g12[g] = reinterpret_cast<GemmJob*>(d.mem + o_g12[g]);
    d.g3[g] = reinterpret_cast<GemmJob*>(d.mem + o_g3[g]);
    d.n_g12[g] = (int)t.g12_jobs[g].size();
    d.n_g3[g] = (int)t.g3_jobs[g].size();
    d.flops_g1[g] = t.flops_g1[g];
    d.flops_g2[g] = t.flops_g2[g];
    d.flops_g3[g] = t.flops_g3[g];
  }
  d.mom_mats = reinterpret_cast<MomMat*>(d.mem + o_mm);
  d.mom_blocks = reinterpret_cast<MomBlock*>(d.mem + o_mb);
  d.hook_mats = reinterpret_cast<HookMat*>(d.mem + o_hm);
  d.hook_blocks = reinterpret_cast<HookBlock*>(d.mem + o_hb);
  d.hook1_blocks = reinterpret_cast<HookBlock*>(d.mem + o_hb1);
  d.n_hook1 = (int)t.hook1_blocks.size();
  d.tile_mats = reinterpret_cast<TileMat*>(d.mem + o_tm);
  d.tile_jobs = reinterpret_cast<TileJob*>(d.mem + o_tj);
  d.n_tile = (int)t.tile_jobs.size();
  d.tile_groups = t.tile_groups;
  d.flops_tile = t.flops_tile;
  d.bytes_tile = t.bytes_tile;
  d.nparts = reinterpret_cast<int32_t*>(d.mem + o_np);
  d.part_base = reinterpret_cast<int64_t*>(d.mem + o_pb);
  d.n_mom = (int)t.mom_blocks.size();
  d.n_hook = (int)t.hook_blocks.size();
  d.parts_total = t.parts_total;
  d.nslots = (int)t.nparts.size();
  d.nunits = (int)t.units.size();
  d.nmats = (int)((t.nparts.size() - t.units.size()) / 2);
  d.bytes_mom = t.bytes_mom;
  d.bytes_hook1 = t.bytes_hook1;
  d.bytes_hook2 = t.bytes_hook2;
  d.bytes_sumsq = t.bytes_sumsq;
}


int upload_chunk(State& st, const ChunkTables& t, DevTables& d, hipStream_t s) {
  std::vector<char> blob;
  BlobOffsets o;
  serialize_chunk(t, blob, o);
  // Once per new (buffers, shapes, options) set: device memory from the
  // stream-ordered allocator and a copy from pinned staging, both queued on
  // the caller's stream, so the host does not wait for earlier work.
  Staging* sg = nullptr;
  for (auto& c : st.staging)
    if (c.cap >= blob.size() && hipEventQuery(c.done) == hipSuccess) {
      sg = &c;
      break;
    }
  if (!sg) {
    Staging n;
    n.cap = std::max<size_t>(blob.size(), (size_t)1 << 20);
    if (hipHostMalloc((void**)&n.p, n.cap, hipHostMallocDefault) != hipSuccess) return MUONH_ENOMEM;
    if (hipEventCreateWithFlags(&n.done, hipEventDisableTiming) != hipSuccess) {
      (void)hipHostFree(n.p);
      return MUONH_EHIP;
    }
    st.staging.push_back(n);
    sg = &st.staging.back();
  }
  memcpy(sg->p, blob.data(), blob.size());
  char* mem = nullptr;
  if (hipMallocAsync((void**)&mem, blob.size(), s) == hipSuccess) {
    d.mem_async = true;
  } else {
    (void)hipGetLastError();
    mem = nullptr;
    if (hipMalloc(&mem, blob.size()) != hipSuccess) return MUONH_ENOMEM;
  }
  d.mem = mem;
  if (hipMemcpyAsync(mem, sg->p, blob.size(), hipMemcpyHostToDevice, s) != hipSuccess) return MUONH_EHIP;
  if (hipEventRecord(sg->done, s) != hipSuccess) return MUONH_EHIP;
  bind_chunk(t, o, mem, d);
  return MUONH_OK;
}

void key_push_ptrs(std::vector<uint64_t>& k, const void* const* a, int n) {
  for (int i = 0; i < n; ++i) k.push_back(a ? (uint64_t)(uintptr_t)a[i] : 0);
}

// Looks up or builds the device tables for this call.
int get_plan(State& st, const Plan& plan, const Cfg& cfg, const CallPtrs& p, const int64_t* shapes,
             hipStream_t s, CachedPlan*& out) {
  std::vector<uint64_t> key;
  key.push_back((uint64_t)cfg.kind);
  key.push_back((uint64_t)cfg.n);
  key.push_back((uint64_t)cfg.tile_T);
  key.push_back(cfg.tile_sizes ? 1 : 0);
  if (cfg.tile_sizes)
    for (int i = 0; i < cfg.n; ++i) key.push_back((uint64_t)(uint32_t)cfg.tile_sizes[i]);
  key.push_back((uint64_t)cfg.state_dt);
  key.push_back((uint64_t)cfg.op_dt);
  key.push_back((uint64_t)cfg.x32);
  key.push_back((uint64_t)cfg.h16);
  key.push_back((uint64_t)cfg.seed32);
  key.push_back((uint64_t)cfg.hook);
  key.push_back((uint64_t)cfg.hb_radius);
  key.push_back((uint64_t)plan.chunks.size());
  key.push_back((uint64_t)plan.lanes);
  for (const auto& c : plan.chunks) key.push_back((uint64_t)c.m1);
  key.push_back((uint64_t)(uintptr_t)st.ws);
  for (int i = 0; i < 2 * cfg.n; ++i) key.push_back((uint64_t)shapes[i]);
  key_push_ptrs(key, p.params, cfg.kind == CALL_NS ? 0 : cfg.n);
  key_push_ptrs(key, p.grads, cfg.n);
  key_push_ptrs(key, p.moms, (cfg.kind == CALL_STEP || cfg.kind == CALL_ADAM) ? cfg.n : 0);
  key_push_ptrs(key, p.vs, cfg.kind == CALL_ADAM ? cfg.n : 0);
  key_push_ptrs(key, p.outs, cfg.kind == CALL_NS ? cfg.n : 0);
  if (p.rho && cfg.kind != CALL_NS) {
    for (int i = 0; i < cfg.n; ++i) {
      uint32_t b;
      memcpy(&b, &p.rho[i], 4);
      key.push_back(b);
    }
  }
  for (auto it = st.plans.begin(); it != st.plans.end(); ++it) {
    if (it->key == key) {
      st.plans.splice(st.plans.begin(), st.plans, it);
      out = &st.plans.front();
      return MUONH_OK;
    }
  }
  CachedPlan cp;
  cp.key = std::move(key);
  cp.lanes = plan.lanes;
  for (size_t c = 0; c < plan.chunks.size(); ++c) {
    ChunkTables t;
    fill_chunk(plan, (int)c, cfg, p, st.ws, t);
    DevTables d;
    const int rc = upload_chunk(st, t, d, s);
    if (rc != MUONH_OK) {
      cp.chunks.push_back(d);
      free_plan(cp, s, true);
      return rc;
    }
    if (plan.lanes > 1) {  // concurrent chunks: disjoint reduction slots
      d.part_off = cp.max_parts;
      d.slot_off = cp.max_slots;
      cp.max_parts += d.parts_total;
      cp.max_slots += d.nslots;
    } else {
      cp.max_parts = std::max(cp.max_parts, d.parts_total);
      cp.max_slots = std::max(cp.max_slots, d.nslots);
    }
    cp.chunks.push_back(d);
  }
  const int rc = ensure_meta(st, cp.max_parts, cp.max_slots);
  if (rc != MUONH_OK) {
    free_plan(cp, s, true);
    return rc;
  }
  st.plans.push_front(std::move(cp));
  while (st.plans.size() > kPlanCacheSize) {
    // bounded cache: the evicted tables are released after the work queued
    // so far on this stream (which, by the calling convention, includes every
    // earlier call's work that may read them)
    free_plan(st.plans.back(), s, true);
    st.plans.pop_back();
  }
  out = &st.plans.front();
  return MUONH_OK;
}

// ------------------------------------------------------------------ profiling
struct Prof {
  State& st;
  hipStream_t s;
  int cls;
  double flops, bytes;
  hipEvent_t e0{}, e1{};
  bool on;
  Prof(State& st_, hipStream_t s_, int cls_, double f, double b)
      : st(st_), s(s_), cls(cls_), flops(f), bytes(b), on(st_.profiling) {
    if (on) {
      (void)hipEventCreate(&e0);
      (void)hipEventCreate(&e1);
      (void)hipEventRecord(e0, s);
    }
  }
  ~Prof() {
    if (on) {
      (void)hipEventRecord(e1, s);
      st.prof.push_back({cls, e0, e1, flops, bytes});
    }
  }
};

// Where a call's reductions and flag counters live: the library's grown
// buffers (regular calls) or the static scratch (muonh_step_noalloc).
struct Meta {
  double* partials;
  double* sums;
  Flags* flags;
};

SlotTable slot_table(const Meta& m, const DevTables& d) {
  SlotTable t;
  t.partials = m.partials + 2 * d.part_off;
  t.nparts = d.nparts;
  t.part_base = d.part_base;
  t.sums = m.sums + 2 * (int64_t)d.slot_off;
  return t;
}

// Last HIP failure, for muonh_last_error().
thread_local char g_last_error[256] = "";

int hip_fail(hipError_t e, const char* what) {
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
  return MUONH_EHIP;
}

#define MUONH_TRY_HIP(x)                                  \
  do {                                                    \
    const hipError_t e_ = (x);                            \
    if (e_ != hipSuccess) return hip_fail(e_, #x);        \
  } while (0)

// Device addresses of the static symbols on one GPU, looked up once per
// device with that device current.
constexpr int kMaxDevices = 64;
struct DevSyms {
  char* scratch = nullptr;
  Flags* flags = nullptr;
};
DevSyms g_syms[kMaxDevices];

int device_symbols(int dev, DevSyms*& out) {
  if (dev < 0 || dev >= kMaxDevices) return MUONH_EINVAL;
  DevSyms& d = g_syms[dev];
  if (d.flags == nullptr) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    void* f = nullptr;
    e = hipGetSymbolAddress(&f, HIP_SYMBOL(g_flags));
    if (e != hipSuccess || f == nullptr) return hip_fail(e, "hipGetSymbolAddress(g_flags)");
    d.scratch = static_cast<char*>(p);
    d.flags = static_cast<Flags*>(f);
  }
  out = &d;
  return MUONH_OK;
}

// Newton-Schulz iteration k of a chunk (K == 0: the single O = X0/||X0||
// pass): G1, G2, G3 over every unit; the last one ends with the finalize of
// the matrices' O-norm slots (||O||^2; for matrices run as resident tiles the
// slot also carries <W, O>).
int run_ns_iter(State& st, const Cfg& cfg, const DevTables& d, const Resolved& r, const SlotTable& sl, hipStream_t s,
                int k) {
  const float eps = r.o.ns_eps;
  if (cfg.K == 0) {
    for (int g = 0; g < kGemmCfgs; ++g) {
      Prof pf(st, s, PC_G3, 0, 0);
      MUONH_TRY_HIP(launch_ns_gemm(cfg.op_dt, cfg.op_dt, 2, g, d.units, d.g3[g], d.n_g3[g], 1.f, 0.f, 0.f, eps, 1,
                                   1, 0, 1, cfg.x32, cfg.seed32, sl, s));
    }
  } else {
    const float a = r.coeffs[3 * k], b = r.coeffs[3 * k + 1], c = r.coeffs[3 * k + 2];
    const int first = k == 0, last = k == cfg.K - 1, cur = k & 1;
    // Storage of this iteration's operands and products: with fp16 iterates
    // (h16) the first iteration reads X0 and forms A0, B0 in bf16 and stores
    // X1 in fp16; every later product reads and stores fp16.
    const int in_dt = (cfg.h16 && !first) ? DT_F16 : cfg.op_dt;
    const int x_dt = cfg.h16 ? DT_F16 : cfg.op_dt;
    for (int g = 0; g < kGemmCfgs; ++g) {
      if (!d.n_g12[g]) continue;
      Prof pf(st, s, PC_G1, d.flops_g1[g], 0);
      MUONH_TRY_HIP(launch_ns_gemm(in_dt, in_dt, 0, g, d.units, d.g12[g], d.n_g12[g], a, b, c, eps, first, 0, cur,
                                   0, cfg.x32, cfg.seed32, sl, s));
    }
    for (int g = 0; g < kGemmCfgs; ++g) {
      if (!d.n_g12[g]) continue;
      Prof pf(st, s, PC_G2, d.flops_g2[g], 0);
      MUONH_TRY_HIP(launch_ns_gemm(in_dt, in_dt, 1, g, d.units, d.g12[g], d.n_g12[g], a, b, c, eps, first, 0, cur,
                                   0, cfg.x32, cfg.seed32, sl, s));
    }
    for (int g = 0; g < kGemmCfgs; ++g) {
      if (!d.n_g3[g]) continue;
      Prof pf(st, s, PC_G3, d.flops_g3[g], 0);
      MUONH_TRY_HIP(launch_ns_gemm(in_dt, last ? in_dt : x_dt, 2, g, d.units, d.g3[g], d.n_g3[g], a, b, c, eps,
                                   first, last, cur, 0, cfg.x32, cfg.seed32, sl, s));
    }
    if (!last) return MUONH_OK;
  }
  Prof pf(st, s, PC_FIN, 0, 0);
  // ||O||^2 per matrix (resident-tile matrices: with <W, O>)
  MUONH_TRY_HIP(launch_finalize(sl, d.nunits, d.nmats, s));
  return MUONH_OK;
}

// Newton-Schulz iterations a chunk runs through the GEMM engine (0: none).
int ns_stage_count(int kind, const Cfg& cfg, const DevTables& d) {
  return (!no_ns(kind) && d.n_mom > 0) ? std::max(cfg.K, 1) : 0;
}

// A step whose matrices all run on the resident-tile kernels, which sum the
// hook's norms where they store O: the hook sums are finalized together with
// the O norms, right after the tile launch.
bool hook_sums_with_tiles(int kind, const Cfg& cfg, const DevTables& d) {
  return kind == CALL_STEP && cfg.hook != kModeNone && d.n_tile > 0 && d.n_mom == 0 && d.n_hook1 == 0;
}

// Stages of one chunk's step: 0 = the opening pass, 1..n = the Newton-Schulz
// iterations through the GEMM engine, n + 1 = the closing passes.
int chunk_stages(int kind, const Cfg& cfg, const DevTables& d) { return 2 + ns_stage_count(kind, cfg, d); }

// One stage of a chunk's step on stream s (see chunk_stages).  When
// rec_open is set it is recorded after the opening pass (momentum and its
// norms, or the resident-tile kernel): the point where the next lane may
// start.
int run_chunk_stage(State& st, const Meta& meta, int kind, const Cfg& cfg, const DevTables& d, const Resolved& r,
                    const CallPtrs& p, float beta, hipStream_t s, int stage, hipEvent_t rec_open) {
  const SlotTable sl = slot_table(meta, d);
  const int nk = ns_stage_count(kind, cfg, d);
  if (stage >= 1 && stage <= nk) return run_ns_iter(st, cfg, d, r, sl, s, stage - 1);
  if (stage == 0) {
    if (!no_ns(kind)) {
      const bool gemm = d.n_mom > 0;  // matrices whose units go through the GEMM engine
      if (d.n_tile > 0) {
        // Hierarchical Muon, resident tiles: momentum, norms and every
        // Newton-Schulz iteration in one launch per tile side.
        TileArgs ta{};
        for (int k = 0; k < cfg.K; ++k)
          for (int j = 0; j < 3; ++j) ta.abc[k][j] = r.coeffs[3 * k + j];
        ta.K = cfg.K;
        // resident tiles keep X in registers: an fp32 master unless X is to be
        // rounded to bf16 between iterations (FOLD); the fused 256-tile kernel
        // always holds it as bf16 (it has no room for more)
        const int fold_res = (cfg.op_dt == DT_BF16 && !cfg.x32 && !cfg.h16) ? 1 : 0;
        ta.beta = beta;
        ta.gcoef = (kind == CALL_STEP && r.o.momentum_ema) ? 1.f - beta : 1.f;
        ta.nesterov = (kind == CALL_STEP && r.o.nesterov) ? 1 : 0;
        ta.eps = r.o.ns_eps;
        ta.st = sl;
        for (const TileGroup& g : d.tile_groups) {
          ta.T = g.T;
          ta.fold = g.T > kTileResidentMax ? 1 : fold_res;
          Prof pf(st, s, g.T > kTileResidentMax ? PC_T256 : PC_TILE, g.flops, g.bytes);
          MUONH_TRY_HIP(launch_tile_ns(cfg.state_dt, cfg.op_dt, d.tile_mats, d.tile_jobs + g.job0, g.njobs, ta, s));
        }
        if (!gemm) {
          // ||O||^2 (and <W, O>) per matrix, and with them the hook's
          // (0, ||W||^2) sums when every matrix summed its norms where O was
          // stored (the next slots; the closing passes then have nothing to
          // reduce): one launch
          Prof pf(st, s, PC_FIN, 0, 0);
          MUONH_TRY_HIP(launch_finalize(sl, d.nunits, hook_sums_with_tiles(kind, cfg, d) ? 2 * d.nmats : d.nmats, s));
        }
      }
      if (gemm) {
        {
          Prof pf(st, s, PC_MOM, 0, d.bytes_mom);
          const bool stp = kind == CALL_STEP;
          MUONH_TRY_HIP(launch_momentum_prep(cfg.state_dt, cfg.op_dt, d.mom_mats, d.mom_blocks, d.n_mom, d.units,
                                             sl, stp ? beta : 0.f, (stp && r.o.momentum_ema) ? 1.f - beta : 1.f,
                                             (stp && r.o.nesterov) ? 1 : 0, s));
        }
        Prof pf(st, s, PC_FIN, 0, 0);
        MUONH_TRY_HIP(launch_finalize(sl, 0, d.nunits, s));  // ||M||^2 per unit
      }
    }
    if (rec_open) MUONH_TRY_HIP(hipEventRecord(rec_open, s));
    return MUONH_OK;
  }
  // closing passes
  if (kind == CALL_ADAM) {
    // AdamH: moments and norms, the per-matrix sums, then the hook
    const bool sums = cfg.hook != kModeNone;
    {
      Prof pf(st, s, PC_AM, 0, d.bytes_hook1);
      MUONH_TRY_HIP(launch_adam_moments(cfg.state_dt, sums, d.hook_mats, d.hook_blocks, d.n_hook, sl, p.adam, s));
    }
    if (sums) {
      Prof pf(st, s, PC_FIN, 0, 0);
      MUONH_TRY_HIP(launch_finalize(sl, d.nunits, 2 * d.nmats, s));  // (||U||^2, <W,U>), (0, ||W||^2)
    }
    Prof pf(st, s, PC_AW, 0, d.bytes_hook2);
    const float decay = cfg.hook == kModeNone ? 1.f - p.eta * r.o.weight_decay : 1.f;
    MUONH_TRY_HIP(launch_adam_write(cfg.hook, d.hook_mats, d.hook_blocks, d.n_hook, sl, p.adam, p.eta,
                                    r.o.zero_rel_eps, r.o.outward, r.o.inward, r.o.rb_eps, decay, meta.flags, s));
    return MUONH_OK;
  }
  if (kind == CALL_PROJ && p.grads) {
    Prof pf(st, s, PC_SQ, 0, d.bytes_sumsq);
    MUONH_TRY_HIP(launch_sumsq(d.hook_mats, d.hook_blocks, d.n_hook, sl, s));
    MUONH_TRY_HIP(launch_finalize(sl, d.nunits, d.nmats, s));  // ||U||^2 per matrix
  }
  if (kind != CALL_NS) {
    if (cfg.hook != kModeNone) {  // Muon's own update needs no norms
      if (d.n_hook1 > 0) {  // matrices whose norms were not summed where O was stored
        Prof pf(st, s, PC_HR, 0, d.bytes_hook1);
        MUONH_TRY_HIP(launch_hook_reduce(cfg.hook, d.hook_mats, d.hook1_blocks, d.n_hook1, sl, p.eta, s));
      }
      if (!hook_sums_with_tiles(kind, cfg, d)) {
        Prof pf(st, s, PC_FIN, 0, 0);
        MUONH_TRY_HIP(launch_finalize(sl, d.nunits + d.nmats, d.nmats, s));  // hook sums per matrix
      }
    }
    {
      Prof pf(st, s, PC_HW, 0, d.bytes_hook2);
      const float decay = cfg.hook == kModeNone ? 1.f - p.eta * r.o.weight_decay : 1.f;
      MUONH_TRY_HIP(launch_hook_write(cfg.hook, d.hook_mats, d.hook_blocks, d.n_hook, sl, p.eta,
                                      r.o.zero_rel_eps, r.o.outward, r.o.inward, r.o.rb_eps, decay, meta.flags,
                                      s));
    }
  }
  return MUONH_OK;
}

int run_call(int kind, const int64_t* shapes, int n, int K, int tile_T, const Resolved& r,
             const CallPtrs& p, float beta) {
  State& st = S();
  std::lock_guard<std::mutex> lk(st.mu);
  int dev = 0;
  MUONH_TRY_HIP(hipGetDevice(&dev));
  if (st.device != -1 && st.device != dev) return MUONH_EINVAL;  // one device per process
  st.device = dev;
  DevSyms* syms = nullptr;
  int rc0 = device_symbols(dev, syms);
  if (rc0 != MUONH_OK) return rc0;
  const size_t limit = r.o.workspace_limit ? r.o.workspace_limit : default_limit();
  Cfg cfg = make_cfg(kind, n, K, tile_T, r, limit);
  Plan plan;
  int rc = make_plan(shapes, cfg, plan);
  if (rc != MUONH_OK) return rc;
  rc = ensure_ws(st, std::max<int64_t>(plan.ws_bytes, 256));
  if (rc != MUONH_OK) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(r.o.stream);
  CachedPlan* cp = nullptr;
  rc = get_plan(st, plan, cfg, p, shapes, s, cp);
  if (rc != MUONH_OK) return rc;
  const Meta meta{st.partials, st.sums, syms->flags};
  if (cp->lanes > 1) {
    // Lane 0 runs on the caller's stream, lane l on the library's side
    // stream l, started after lane l-1's opening pass (and so after all
    // earlier work on s); the lanes then run freely side by side, and s
    // waits for every lane before anything queued after this call.
    const int L = cp->lanes;
    for (int l = 0; l < L; ++l) {
      if (!st.ev_gate[l]) MUONH_TRY_HIP(hipEventCreateWithFlags(&st.ev_gate[l], hipEventDisableTiming));
      if (!st.ev_join[l]) MUONH_TRY_HIP(hipEventCreateWithFlags(&st.ev_join[l], hipEventDisableTiming));
      if (l > 0 && !st.side[l]) MUONH_TRY_HIP(hipStreamCreateWithFlags(&st.side[l], hipStreamNonBlocking));
    }
    // Submission is interleaved stage by stage, so that the side lanes'
    // launches are queued as early as the caller's lane's (queued whole, one
    // lane after the other, a lane would wait for the host to submit the
    // lanes before it).
    int nst = 0;
    for (int l = 0; l < L; ++l) nst = std::max(nst, chunk_stages(kind, cfg, cp->chunks[l]));
    for (int stage = 0; stage < nst; ++stage)
      for (int l = 0; l < L; ++l) {
        const DevTables& d = cp->chunks[l];
        if (stage >= chunk_stages(kind, cfg, d)) continue;
        hipStream_t ls = l == 0 ? s : st.side[l];
        if (stage == 0 && l > 0) MUONH_TRY_HIP(hipStreamWaitEvent(ls, st.ev_gate[l - 1], 0));
        rc = run_chunk_stage(st, meta, kind, cfg, d, r, p, beta, ls, stage,
                             stage == 0 && l + 1 < L ? st.ev_gate[l] : nullptr);
        if (rc != MUONH_OK) return rc;
      }
    for (int l = 1; l < L; ++l) {
      MUONH_TRY_HIP(hipEventRecord(st.ev_join[l], st.side[l]));
      MUONH_TRY_HIP(hipStreamWaitEvent(s, st.ev_join[l], 0));
    }
    return MUONH_OK;
  }
  for (const DevTables& d : cp->chunks)
    for (int stage = 0; stage < chunk_stages(kind, cfg, d); ++stage) {
      rc = run_chunk_stage(st, meta, kind, cfg, d, r, p, beta, s, stage, nullptr);
      if (rc != MUONH_OK) return rc;
    }
  return MUONH_OK;
}

// muonh_step with every device byte in the static scratch: workspace,
// descriptor tables and reduction partials are carved from this GPU's copy of
// the array, the tables go up with one stream-ordered copy, and all work runs
// on the caller's stream (one lane, no side streams or events).  Nothing is
// cached: each call plans and uploads afresh.
int run_step_noalloc(const int64_t* shapes, int n, int K, int tile_T, Resolved r, const CallPtrs& p, float beta) {
  State& st = S();
  std::lock_guard<std::mutex> lk(st.mu);
  r.o.lanes = 1;
  // a quarter of the scratch stays free for the tables and reductions
  Cfg cfg = make_cfg(CALL_STEP, n, K, tile_T, r, kNoAllocScratchBytes / 4 * 3);
  Plan plan;
  int rc = make_plan(shapes, cfg, plan);
  if (rc == MUONH_ENOMEM) {
    snprintf(g_last_error, sizeof(g_last_error),
             "muonh_step_noalloc: one matrix needs more workspace than the %zu bytes the static scratch "
             "(%zu bytes) leaves for it", kNoAllocScratchBytes / 4 * 3, kNoAllocScratchBytes);
    return rc;
  }
  if (rc != MUONH_OK) return rc;
  const int64_t ws_bytes = align256(std::max<int64_t>(plan.ws_bytes, 256));
  int dev = 0;
  MUONH_TRY_HIP(hipGetDevice(&dev));
  if (st.device != -1 && st.device != dev) return MUONH_EINVAL;  // one device per process
  DevSyms* syms = nullptr;
  rc = device_symbols(dev, syms);
  if (rc != MUONH_OK) return rc;
  st.device = dev;
  char* const base = syms->scratch;
  // layout: [workspace | tables of every chunk | slot sums | partials]
  const size_t nch = plan.chunks.size();
  std::vector<ChunkTables> tabs(nch);
  std::vector<BlobOffsets> offs(nch);
  std::vector<char>& blob = st.noalloc_blob;
  blob.clear();
  int64_t max_parts = 1;
  int max_slots = 1;
  for (size_t c = 0; c < nch; ++c) {
    fill_chunk(plan, (int)c, cfg, p, base, tabs[c]);
    serialize_chunk(tabs[c], blob, offs[c]);
    max_parts = std::max(max_parts, tabs[c].parts_total);
    max_slots = std::max(max_slots, (int)tabs[c].nparts.size());
  }
  const int64_t tables_off = ws_bytes;
  const int64_t sums_off = tables_off + align256((int64_t)blob.size());
  const int64_t parts_off = sums_off + align256((int64_t)max_slots * 2 * (int64_t)sizeof(double));
  const int64_t total = parts_off + align256(max_parts * 2 * (int64_t)sizeof(double));
  if (total > (int64_t)kNoAllocScratchBytes) {
    snprintf(g_last_error, sizeof(g_last_error),
             "muonh_step_noalloc: the call needs %lld bytes of scratch, the static scratch holds %zu",
             (long long)total, kNoAllocScratchBytes);
    return MUONH_ENOMEM;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(r.o.stream);
  // stream-ordered: earlier work on s that still reads the scratch finishes first
  MUONH_TRY_HIP(hipMemcpyAsync(base + tables_off, blob.data(), blob.size(), hipMemcpyHostToDevice, s));
  const Meta meta{reinterpret_cast<double*>(base + parts_off), reinterpret_cast<double*>(base + sums_off),
                  syms->flags};
  for (size_t c = 0; c < nch; ++c) {
    DevTables d;
    bind_chunk(tabs[c], offs[c], base + tables_off, d);
    for (int stage = 0; stage < chunk_stages(CALL_STEP, cfg, d); ++stage) {
      rc = run_chunk_stage(st, meta, CALL_STEP, cfg, d, r, p, beta, s, stage, nullptr);
      if (rc != MUONH_OK) return rc;
    }
  }
  return MUONH_OK;
}

bool bad_ptrs(const void* const* a, int n) {
  if (!a) return true;
  for (int i = 0; i < n; ++i)
    if (!a[i]) return true;
  return false;
}

int validate_common(const int64_t* shapes, int n, int K, int tile_T) {
  if (!shapes || n <= 0) return MUONH_EINVAL;
  if (K < 0 || K > kMaxK) return MUONH_EINVAL;
  for (int i = 0; i < 2 * n; ++i)
    if (shapes[i] < 1) return MUONH_EINVAL;
  return check_tile(tile_T);
}

}  // namespace
}  // namespace muonh

using namespace muonh;

extern "C" {

void muonh_default_opts(muonh_opts* o) {
  if (!o) return;
  memset(o, 0, sizeof(*o));
  o->stream = nullptr;
  o->state_dtype = MUONH_BF16;
  o->ns_dtype = MUONH_BF16;
  o->ns_precision = MUONH_NS_H16;
  o->coeffs = nullptr;
  o->ns_eps = 1e-7f;
  o->zero_rel_eps = 1e-6f;
  o->hook = MUONH_HOOK_HYPERBALL;
  o->outward = 0.5f;
  o->inward = 1.0f;
  o->rb_eps = 1e-15f;
  o->workspace_limit = 0;
  o->momentum_ema = 0;
  o->nesterov = 0;
  o->weight_decay = 0.f;
  o->lanes = 0;
  o->hyperball_step = MUONH_HB_STEP_UNIT;
  o->tile_sizes = nullptr;
  o->param_dtype = MUONH_F32;
  o->deterministic = 1;
}

int muonh_step(void* const params[], const void* const grads[], void* const moms[], const int64_t shapes[],
               int n, float eta, float beta, int K, const float rho[], int tile_T, const muonh_opts* opts) {
  int rc = validate_common(shapes, n, K, tile_T);
  if (rc != MUONH_OK) return rc;
  if (bad_ptrs(params, n) || bad_ptrs(grads, n) || bad_ptrs((const void* const*)moms, n)) return MUONH_EINVAL;
  if (!std::isfinite(eta) || eta < 0.f) return MUONH_EINVAL;
  if (!std::isfinite(beta) || beta < 0.f || beta >= 1.f) return MUONH_EINVAL;
  Resolved r;
  rc = resolve(opts, K, r);
  if (rc != MUONH_OK) return rc;
  rc = check_tile_sizes(r.o.tile_sizes, n);
  if (rc != MUONH_OK) return rc;
  if (r.o.hook == MUONH_HOOK_HYPERBALL) {
    if (!rho) return MUONH_EINVAL;
    for (int i = 0; i < n; ++i)
      if (!std::isfinite(rho[i]) || rho[i] <= 0.f) return MUONH_EINVAL;
  }
  for (int i = 0; i < n; ++i)
    if (grads[i] == moms[i]) return MUONH_EINVAL;
  CallPtrs p{params, grads, moms, nullptr, r.o.hook == MUONH_HOOK_HYPERBALL ? rho : nullptr, eta};
  return run_call(CALL_STEP, shapes, n, K, tile_T, r, p, beta);
}

int muonh_step_noalloc(void* const params[], const void* const grads[], void* const moms[],
                       const int64_t shapes[], int n, float eta, float beta, int K, const float rho[], int tile_T,
                       const muonh_opts* opts) {
  int rc = validate_common(shapes, n, K, tile_T);
  if (rc != MUONH_OK) return rc;
  if (bad_ptrs(params, n) || bad_ptrs(grads, n) || bad_ptrs((const void* const*)moms, n)) return MUONH_EINVAL;
  if (!std::isfinite(eta) || eta < 0.f) return MUONH_EINVAL;
  if (!std::isfinite(beta) || beta < 0.f || beta >= 1.f) return MUONH_EINVAL;
  Resolved r;
  rc = resolve(opts, K, r);
  if (rc != MUONH_OK) return rc;
  rc = check_tile_sizes(r.o.tile_sizes, n);
  if (rc != MUONH_OK) return rc;
  if (r.o.hook == MUONH_HOOK_HYPERBALL) {
    if (!rho) return MUONH_EINVAL;
    for (int i = 0; i < n; ++i)
      if (!std::isfinite(rho[i]) || rho[i] <= 0.f) return MUONH_EINVAL;
  }
  for (int i = 0; i < n; ++i)
    if (grads[i] == moms[i]) return MUONH_EINVAL;
  CallPtrs p{params, grads, moms, nullptr, r.o.hook == MUONH_HOOK_HYPERBALL ? rho : nullptr, eta};
  return run_step_noalloc(shapes, n, K, tile_T, r, p, beta);
}

int adamh_step(void* const params[], const void* const grads[], void* const exp_avg[], void* const exp_avg_sq[],
               const int64_t shapes[], int n, float eta, float beta1, float beta2, float eps, int64_t step,
               const float rho[], const muonh_opts* opts) {
  if (!shapes || n <= 0) return MUONH_EINVAL;
  for (int i = 0; i < 2 * n; ++i)
    if (shapes[i] < 1) return MUONH_EINVAL;
  if (bad_ptrs(params, n) || bad_ptrs(grads, n) || bad_ptrs((const void* const*)exp_avg, n) ||
      bad_ptrs((const void* const*)exp_avg_sq, n))
    return MUONH_EINVAL;
  if (!std::isfinite(eta) || eta < 0.f) return MUONH_EINVAL;
  if (!std::isfinite(beta1) || beta1 < 0.f || beta1 >= 1.f) return MUONH_EINVAL;
  if (!std::isfinite(beta2) || beta2 < 0.f || beta2 >= 1.f) return MUONH_EINVAL;
  if (!std::isfinite(eps) || eps <= 0.f || step < 1) return MUONH_EINVAL;
  Resolved r;
  int rc = resolve(opts, 0, r);
  if (rc != MUONH_OK) return rc;
  if (r.o.hook == MUONH_HOOK_HYPERBALL) {
    if (!rho) return MUONH_EINVAL;
    for (int i = 0; i < n; ++i)
      if (!std::isfinite(rho[i]) || rho[i] <= 0.f) return MUONH_EINVAL;
  }
  for (int i = 0; i < n; ++i)
    if (exp_avg[i] == exp_avg_sq[i] || grads[i] == exp_avg[i] || grads[i] == exp_avg_sq[i]) return MUONH_EINVAL;
  CallPtrs p{params, grads, exp_avg, nullptr, r.o.hook == MUONH_HOOK_HYPERBALL ? rho : nullptr, eta};
  p.vs = exp_avg_sq;
  // bias corrections in double, from the step count
  const double bc1 = 1.0 - std::pow((double)beta1, (double)step), bc2 = 1.0 - std::pow((double)beta2, (double)step);
  if (!(bc1 > 0.0) || !(bc2 > 0.0)) return MUONH_EINVAL;
  p.adam = AdamArgs{beta1, beta2, (float)(1.0 / bc1), (float)(1.0 / bc2), eps};
  return run_call(CALL_ADAM, shapes, n, 0, 0, r, p, 0.f);
}

int ns_orthogonalize(const void* const in[], void* const out[], const int64_t shapes[], int n, int K,
                     int tile_T, const muonh_opts* opts) {
  int rc = validate_common(shapes, n, K, tile_T);
  if (rc != MUONH_OK) return rc;
  if (bad_ptrs(in, n) || bad_ptrs((const void* const*)out, n)) return MUONH_EINVAL;
  Resolved r;
  rc = resolve(opts, K, r);
  if (rc != MUONH_OK) return rc;
  rc = check_tile_sizes(r.o.tile_sizes, n);
  if (rc != MUONH_OK) return rc;
  CallPtrs p{nullptr, in, nullptr, out, nullptr, 0.f};
  return run_call(CALL_NS, shapes, n, K, tile_T, r, p, 0.f);
}

int frob_project(void* const W[], const void* const U[], const int64_t shapes[], int n, float eta,
                 const float rho[], const muonh_opts* opts) {
  if (!shapes || n <= 0) return MUONH_EINVAL;
  for (int i = 0; i < 2 * n; ++i)
    if (shapes[i] < 1) return MUONH_EINVAL;
  if (bad_ptrs((const void* const*)W, n) || !rho) return MUONH_EINVAL;
  if (!std::isfinite(eta) || eta < 0.f) return MUONH_EINVAL;
  for (int i = 0; i < n; ++i)
    if (!std::isfinite(rho[i]) || rho[i] <= 0.f) return MUONH_EINVAL;
  Resolved r;
  int rc = resolve(opts, 0, r);
  if (rc != MUONH_OK) return rc;
  r.o.hook = MUONH_HOOK_HYPERBALL;
  // A NULL U array is the plain projection; NULL entries are zero updates.
  std::vector<const void*> us;
  const void* const* up = nullptr;
  if (U) {
    bool any = false;
    for (int i = 0; i < n; ++i) any = any || U[i];
    if (any) up = U;
  }
  CallPtrs p{W, up, nullptr, nullptr, rho, eta};
  return run_call(CALL_PROJ, shapes, n, 0, 0, r, p, 0.f);
}

int muonh_get_flags(uint64_t out[4]) {
  if (!out) return MUONH_EINVAL;
  State& st = S();
  std::lock_guard<std::mutex> lk(st.mu);
  if (st.device < 0 || g_syms[st.device].flags == nullptr) {
    out[0] = out[1] = out[2] = out[3] = 0;
    return MUONH_OK;
  }
  Flags f;
  if (hipDeviceSynchronize() != hipSuccess) return MUONH_EHIP;
  if (hipMemcpy(&f, g_syms[st.device].flags, sizeof(f), hipMemcpyDeviceToHost) != hipSuccess) return MUONH_EHIP;
  out[0] = f.zero_update;
  out[1] = f.restored;
  out[2] = f.unrestorable;
  out[3] = f.nonfinite;
  return MUONH_OK;
}

int muonh_reset_flags(void) {
  State& st = S();
  std::lock_guard<std::mutex> lk(st.mu);
  if (st.device < 0 || g_syms[st.device].flags == nullptr) return MUONH_OK;
  if (hipDeviceSynchronize() != hipSuccess) return MUONH_EHIP;
  if (hipMemset(g_syms[st.device].flags, 0, sizeof(Flags)) != hipSuccess) return MUONH_EHIP;
  return MUONH_OK;
}

const char* muonh_strerror(int code) {
  switch (code) {
    case MUONH_OK: return "success";
    case MUONH_EINVAL: return "invalid argument";
    case MUONH_ENOMEM: return "workspace limit exceeded or device allocation failed";
    case MUONH_EHIP: return "HIP runtime or kernel launch error";
    case MUONH_ENOTIMPL: return "not implemented by this library";
    default: return "unknown error";
  }
}

void muonh_release(void) {
  State& st = S();
  std::lock_guard<std::mutex> lk(st.mu);
  if (st.device < 0) return;
  (void)hipDeviceSynchronize();
  clear_plans(st);
  if (st.ws) (void)hipFree(st.ws);
  if (st.partials) (void)hipFree(st.partials);
  if (st.sums) (void)hipFree(st.sums);
  if (g_syms[st.device].flags) (void)hipMemset(g_syms[st.device].flags, 0, sizeof(Flags));
  for (void* q : st.retired) (void)hipFree(q);
  st.retired.clear();
  for (auto& g : st.staging) {
    (void)hipEventDestroy(g.done);
    (void)hipHostFree(g.p);
  }
  st.staging.clear();
  for (int l = 0; l < kMaxLanes; ++l) {
    if (st.side[l]) (void)hipStreamDestroy(st.side[l]);
    if (st.ev_gate[l]) (void)hipEventDestroy(st.ev_gate[l]);
    if (st.ev_join[l]) (void)hipEventDestroy(st.ev_join[l]);
    st.side[l] = nullptr;
    st.ev_gate[l] = st.ev_join[l] = nullptr;
  }
  for (auto& r : st.prof) {
    (void)hipEventDestroy(r.e0);
    (void)hipEventDestroy(r.e1);
  }
  st.prof.clear();
  st.profiling = false;
  st.ws = nullptr;
  st.ws_bytes = 0;
  st.partials = nullptr;
  st.partials_cap = 0;
  st.sums = nullptr;
  st.slots_cap = 0;
  st.device = -1;
}

int muonh_plan_query(const int64_t shapes[], int n, int K, int tile_T, const muonh_opts* opts,
                     size_t workspace_limit, int64_t out[7]) {
  if (!out) return MUONH_EINVAL;
  int rc = validate_common(shapes, n, K, tile_T);
  if (rc != MUONH_OK) return rc;
  Resolved r;
  rc = resolve(opts, K, r);
  if (rc != MUONH_OK) return rc;
  rc = check_tile_sizes(r.o.tile_sizes, n);
  if (rc != MUONH_OK) return rc;
  if (workspace_limit == 0) workspace_limit = (size_t)1 << 62;
  Cfg cfg = make_cfg(CALL_STEP, n, K, tile_T, r, workspace_limit);
  Plan plan;
  rc = make_plan(shapes, cfg, plan);
  if (rc != MUONH_OK) return rc;
  out[0] = plan.lanes > 1 ? 1 : (int64_t)plan.chunks.size();
  out[1] = plan.ws_bytes;
  out[2] = plan.units;
  out[3] = (int64_t)plan.ns_flops;
  out[4] = plan.jobs_per_iter;
  out[5] = (int64_t)plan.stream_bytes;
  out[6] = plan.lanes;
  return MUONH_OK;
}

int muonh_profile_begin(void) {
  State& st = S();
  std::lock_guard<std::mutex> lk(st.mu);
  for (auto& r : st.prof) {
    (void)hipEventDestroy(r.e0);
    (void)hipEventDestroy(r.e1);
  }
  st.prof.clear();
  st.profiling = true;
  return MUONH_OK;
}

int muonh_profile_read(muonh_kernel_stat* out, int max, int* n_out) {
  State& st = S();
  std::lock_guard<std::mutex> lk(st.mu);
  st.profiling = false;
  muonh_kernel_stat acc[PC_N];
  memset(acc, 0, sizeof(acc));
  for (int c = 0; c < PC_N; ++c) strncpy(acc[c].name, kClassNames[c], sizeof(acc[c].name) - 1);
  int rc = MUONH_OK;
  for (auto& r : st.prof) {
    if (hipEventSynchronize(r.e1) != hipSuccess) rc = MUONH_EHIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.e0, r.e1) != hipSuccess) rc = MUONH_EHIP;
    acc[r.cls].launches += 1;
    acc[r.cls].total_ms += ms;
    acc[r.cls].flops += r.flops;
    acc[r.cls].bytes += r.bytes;
    (void)hipEventDestroy(r.e0);
    (void)hipEventDestroy(r.e1);
  }
  st.prof.clear();
  int k = 0;
  for (int c = 0; c < PC_N && k < max; ++c)
    if (acc[c].launches) out[k++] = acc[c];
  if (n_out) *n_out = k;
  return rc;
}

const char* muonh_version(void) { return "libmuonh 0.1 (gfx950)"; }

const char* muonh_last_error(void) { return g_last_error; }

}  // extern "C"
