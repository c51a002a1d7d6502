// Plain-old-data descriptors shared by the host planner and the HIP kernels.
// No HIP headers here: the planner builds these tables on the host, copies
// them to the device once per step, and the kernels decode them.
#pragma once
#include <stdint.h>

namespace muonh {

enum DType : int32_t { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };  // DT_F16: Newton-Schulz storage only

// Padding granule of every workspace leading dimension (elements).  Producers
// write zeros into [valid, padded) so GEMM loaders can read whole vectors.
constexpr int kPad = 64;

inline int64_t pad_up(int64_t v, int64_t g) { return (v + g - 1) / g * g; }

// Reduction slots: each slot owns nparts double2 partials starting at
// part_base; producers store one partial per block, a finalize launch sums
// each slot's partials in a fixed order (deterministic) into sums[slot].
struct SlotTable {
  double* partials;        // 2 doubles per partial
  const int32_t* nparts;   // per slot
  const int64_t* part_base;// per slot, index of the first partial
  double* sums;            // 2 doubles per slot
};

// One Newton-Schulz unit: a whole matrix, or one HiMuon tile handled as a
// T x T matrix.  Logical X is r x s with r <= s; it is kept only as X^T:
//   XT layout: ld_s = pad(s) rows of ld_r = pad(r) elements, the padding
//   (rows >= s, columns >= r) zero.
struct NsUnit {
  int32_t r, s;
  int32_t ld_s, ld_r;
  int32_t norm_slot;    // slot holding ||M||^2 for the pre-scale
  int32_t onorm_slot;   // slot collecting ||O||^2 (per full matrix)
  int32_t onorm_part0;  // first partial of this unit inside onorm_slot
  int32_t o_trans;      // 1: X(i, n) is out[n * o_ld + i]; 0: out[i * o_ld + n]
  int32_t o_rows;       // valid rows of X written to out (i < o_rows)
  int32_t o_cols;       // valid cols of X written to out (n < o_cols)
  int32_t o_dtype;      // DType of out
  int32_t g3_cols;      // number of G3 column tiles of this unit (for partial numbering)
  int64_t o_ld;
  void* o_ptr;          // output base, already offset to the unit's origin
  void* xt[2];          // op-dtype X^T ping-pong (XT layout)
  float* x32;           // fp32 X^T (XT layout) or nullptr: the master copy (X32 mode)
                        // and/or the fp32 X0 that seeds the first a X term
  void* a;              // op-dtype A = X X^T (r rows, ld_r)
  void* b;              // op-dtype B = b A + c A A (r rows, ld_r)
};

// One output macro-tile of a grouped GEMM launch.
struct GemmJob {
  int32_t unit;
  int32_t tm, tn;       // macro-tile row / column
  int32_t kchunks;      // K extent in BK steps (for scheduling only)
};

// Momentum / prep: one source matrix.
struct MomMat {
  const void* g;        // gradient (or the NS input for ns_orthogonalize)
  void* m;              // momentum, updated in place; nullptr = prep only (m = g)
  int64_t H, W;         // M layout rows, cols (ld = W)
  int32_t trans;        // full mode: X = M^T (H > W)
  int32_t tile_T;       // 0: full matrix; > 0: per-tile units (multiple of 64)
  int32_t unit0;        // first NsUnit of this matrix
  int32_t ntc;          // tiles per row (tile mode)
  int32_t nbc;          // 64-wide column blocks over the padded extent
  int32_t write_x;      // 1: write X0^T into the units' workspace
  int32_t write_x32;    // 1: also write the fp32 X0^T into the units' x32 buffers
};

// One 64 x 64 block of a momentum / prep launch.
struct MomBlock {
  int32_t mat;
  int32_t br, bc;       // block row / column in the padded M grid
  int32_t slot;         // norm slot this block contributes to (-1: none)
  int32_t part;         // partial index inside the slot
  int32_t pad_;
};

// Hook / projection / norm passes: one full matrix, streamed flat.
struct HookMat {
  float* w;             // fp32 weights (M layout), updated in pass 2
  const void* o;        // update direction (o_dtype), nullptr = zero update;
                        // AdamH: the gradient (o_dtype), the direction is Adam's
  float* am;            // AdamH: first moment (fp32, in place); else nullptr
  float* av;            // AdamH: second moment (fp32, in place); else nullptr
  int64_t numel;
  int32_t o_dtype;
  int32_t onorm_slot;   // slot of ||O||^2 (Hyperball); -1: none (zero update);
                        // AdamH: (||U||^2, <W, U>)
  int32_t slot;         // slot for this matrix's pass-1 sums (AdamH: (0, ||W||^2))
  int32_t nblocks;      // blocks of this matrix in a pass
  float rho;            // Hyperball radius
  float oscale;         // Hyperball: step scale (1, or rho for the radius-sized step);
                        // RadialBrake / plain update: shape scale max(1, H/W)^0.5
  int32_t fused;        // 1: <W, O> and ||W||^2 were summed where O was stored (no pass 1)
  int32_t pad_;
};

struct HookBlock {
  int32_t mat;
  int32_t blk;          // block index within the matrix
};

// Resident-tile Newton-Schulz (Hierarchical Muon with T <= kTileResidentMax):
// one workgroup runs the whole step of one tile.
constexpr int kTileResidentMax = 128;
// Tiles of side kTileResidentMax < T <= kTileFusedMax run on the fused
// 256-tile kernel (bf16 operands and state, X in bf16 between iterations).
constexpr int kTileFusedMax = 256;
constexpr int kTileMaxK = 64;

struct TileMat {
  const void* g;        // gradient; nullptr: m is the Newton-Schulz input itself
  void* m;              // momentum (updated in place when g is set) or NS input
  void* out;            // orthogonalized output (H x W, ld = W)
  int64_t H, W;
  int32_t out_dtype;
  int32_t onorm_slot;   // slot collecting this matrix's ||O||^2 (and <W, O> with w)
  int32_t vec;          // 1: rows and tile origins allow 16-byte accesses
  int32_t hook_slot;    // slot receiving (0, ||W||^2) when w is set
  const float* w;       // weights (H x W, ld = W) or nullptr: the step's hook norms
                        // <W, O> and ||W||^2 are then summed where O is stored
};

struct TileJob {
  int32_t mat;
  int32_t ti, tj;       // tile row / column
  int32_t part;         // partial index inside the matrix's O-norm slot
};

struct TileArgs {
  float abc[kTileMaxK][3];  // (a, b, c) per iteration
  int T;                    // tile side
  int K;                    // iterations
  int fold;                 // 1: round the master X to bf16 after every iteration
  float beta;               // momentum coefficient (used when TileMat::g is set)
  float gcoef;              // weight of G in the buffer update: 1 (sum) or 1 - beta (EMA)
  int nesterov;             // 1: NS input is gcoef*G + beta*M (Nesterov blend)
  float eps;                // pre-scale eps
  SlotTable st;
};

// Hook modes.
constexpr int kModeHB = 0;    // Hyperball
constexpr int kModeRB = 1;    // RadialBrake
constexpr int kModeNone = 2;  // Muon's own update (decoupled weight decay)
constexpr int kModeRel = 3;   // RelativeUpdate (update scaled to ||W||)

// Adam's step constants (AdamH): m <- b1 m + (1 - b1) g,
// v <- b2 v + (1 - b2) g^2, U = (m * ibc1) / (sqrt(v * ibc2) + eps) with the
// bias corrections ibc = 1 / (1 - b^t).
struct AdamArgs {
  float b1, b2, ibc1, ibc2, eps;
};

// Elements per block of the flat hook / norm passes (256 threads x 32).
constexpr int kHookBlockElems = 8192;

// Device-side flag counters (see muonh_get_flags).
struct Flags {
  unsigned long long zero_update;
  unsigned long long restored;
  unsigned long long unrestorable;
  unsigned long long nonfinite;
};

}  // namespace muonh
