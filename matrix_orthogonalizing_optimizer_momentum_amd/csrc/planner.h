// Host-side planning for libmuonh: validation, Newton-Schulz units, memory-
// bounded chunks, GEMM job lists, momentum / hook block lists and reduction
// slots.  Pure host C++ (no HIP runtime calls), so it can be exercised on a
// machine without a GPU through muonh_plan_query.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "desc.h"

namespace muonh {

enum CallKind { CALL_STEP = 0, CALL_NS = 1, CALL_PROJ = 2, CALL_ADAM = 3 };
// Calls with no Newton-Schulz work (pure streaming passes).
inline bool no_ns(int kind) { return kind == CALL_PROJ || kind == CALL_ADAM; }

struct Cfg {
  int kind;
  int n;
  int K;
  int tile_T;
  int state_dt, op_dt;
  int x32;        // fp32 master X (bf16 operands only)
  int h16;        // bf16 operands: X, A, B stored in fp16 after the first product (MUONH_NS_H16)
  int seed32;     // bf16 operands with an NS input that is not a bf16 value (fp32
                  // state, or the Nesterov blend): the first a X term is seeded
                  // from an fp32 copy of X0
  int hook;       // kModeHB / kModeRB / kModeNone / kModeRel
  int hb_radius;  // Hyperball: radius-sized step (eta * rho * U_hat)
  size_t ws_limit;
  int lanes;      // concurrent lanes, 1..kMaxLanes; 0: automatic (see make_plan)
  const int32_t* tile_sizes;  // host, n per-matrix tile sides (0: full matrix); nullptr: tile_T for all
};

// Per source matrix.
struct MatPlan {
  int64_t H, W;
  int T;           // tile side (0: full-matrix Newton-Schulz)
  int r, s;        // full mode: oriented sides; tile mode: T, T
  int trans;       // full mode: H > W
  int nunits;      // 1, or tiles
  int ntr, ntc;    // tile grid (tile mode)
  int64_t ws_bytes;
};

constexpr int kMaxLanes = 4;
// Automatic lanes: two, except for Newton-Schulz on the GEMM engine (full
// matrices, or tiles above the resident size) when one iteration over the
// whole set exceeds this many flops (about 1.5 ms of matrix-core work).
constexpr double kAutoLaneIterFlops = 2e12;

struct ChunkPlan {
  int m0, m1;      // matrices [m0, m1)
  int64_t ws_bytes;
  int64_t ws_off;  // start of this chunk's region in the workspace
};

struct Plan {
  std::vector<MatPlan> mats;
  std::vector<ChunkPlan> chunks;
  int64_t ws_bytes = 0;     // max over chunks (sequential), sum (lanes)
  int lanes = 1;            // > 1: the chunks are concurrent lanes
  int64_t units = 0;
  double ns_flops = 0;      // dense, true sides
  int64_t jobs_per_iter = 0;
  double stream_bytes = 0;  // algorithmic
};

// Byte sizes of one unit's workspace pieces (each rounded to 256 B).
struct UnitBytes {
  int64_t xt, x32, a, b;
  int64_t total() const { return 2 * xt + x32 + a + b; }
};
UnitBytes unit_bytes(int r, int s, int op_dt, int x32);  // x32: an fp32 X^T buffer (master or X0 seed)

inline int64_t align256(int64_t v) { return (v + 255) / 256 * 256; }
inline int esize(int dt) { return dt == DT_F32 ? 4 : 2; }

// Builds mats / chunks; returns MUONH_OK, MUONH_EINVAL or MUONH_ENOMEM.
int make_plan(const int64_t* shapes, const Cfg& cfg, Plan& plan);

// Host tables of one chunk (everything a launch sequence needs).
// GEMM tile configurations: 0 = 128 x 128 output tiles (4 waves, two
// workgroups per CU); 1 = 256 x 256 (8 waves of 64 x 128, one workgroup per
// CU, bf16 operands): a third less LDS traffic per MFMA, for units large
// enough to fill the chip with them.
constexpr int kGemmCfgs = 3;
inline int gemm_tile_side(int cfg) { return cfg == 1 ? 256 : cfg == 2 ? 64 : 128; }
// Configuration of a unit's G1/G2 (phase12) or G3 products.
int unit_gemm_cfg(int r, int op_dt, bool phase12);

// Hierarchical Muon with T <= kTileResidentMax runs on the resident-tile
// kernel (one workgroup per tile for the whole step, momentum fused, no
// workspace but the step's O buffer).  Tiles of side 128 < T <= 256 do the
// same on the 256-tile kernel when X stays bf16 between iterations and the NS
// input is a bf16 value (bf16 operands and state, FOLD, no Nesterov blend);
// otherwise, and for larger tiles, they go through the GEMM engine.
bool tile256_enabled();  // MUONH_TILE256=0 routes such tiles to the GEMM engine (tuning runs)
inline bool fused256_ok(const Cfg& c) {
  return c.op_dt == DT_BF16 && c.state_dt == DT_BF16 && !c.x32 && !c.seed32 && tile256_enabled();
}
inline bool resident_tile(const Cfg& c, int T) {
  return T > 0 && (T <= kTileResidentMax || (T <= kTileFusedMax && fused256_ok(c)));
}
inline int mat_tile(const Cfg& c, int i) { return c.tile_sizes ? c.tile_sizes[i] : c.tile_T; }

// Resident-tile launches of one chunk: one per distinct tile side.
struct TileGroup {
  int T;
  int job0, njobs;
  double flops, bytes;
};

struct ChunkTables {
  std::vector<NsUnit> units;
  std::vector<GemmJob> g12_jobs[kGemmCfgs], g3_jobs[kGemmCfgs];
  std::vector<MomMat> mom_mats;
  std::vector<MomBlock> mom_blocks;
  std::vector<HookMat> hook_mats;
  std::vector<HookBlock> hook_blocks;
  std::vector<TileMat> tile_mats;
  std::vector<TileJob> tile_jobs;
  std::vector<TileGroup> tile_groups;
  std::vector<HookBlock> hook1_blocks;  // pass-1 blocks: matrices whose norms are not fused
  std::vector<int32_t> nparts;
  std::vector<int64_t> part_base;
  int64_t parts_total = 0;
  double flops_g1[kGemmCfgs] = {}, flops_g2[kGemmCfgs] = {}, flops_g3[kGemmCfgs] = {};
  double bytes_mom = 0, bytes_hook1 = 0, bytes_hook2 = 0, bytes_sumsq = 0;
  double flops_tile = 0, bytes_tile = 0;
};

struct CallPtrs {
  void* const* params;        // STEP, PROJ, ADAM
  const void* const* grads;   // STEP, ADAM: grads; NS: inputs; PROJ: U (may be null)
  void* const* moms;          // STEP; ADAM: first moments
  void* const* outs;          // NS
  const float* rho;           // STEP (HB), PROJ, ADAM (HB)
  float eta;
  void* const* vs = nullptr;  // ADAM: second moments
  AdamArgs adam{};            // ADAM
};

// Fill the tables of chunk c; ws is the data workspace base (device).
void fill_chunk(const Plan& plan, int c, const Cfg& cfg, const CallPtrs& p, char* ws, ChunkTables& t);

}  // namespace muonh
