/*
 * muonh.h -- C ABI of libmuonh, the MuonH / Hierarchical-Muon optimizer step
 * for AMD Instinct MI355X (gfx950).
 *
 * One step over a list of weight matrices W_i (H_i x W_i, row-major, fp32
 * master copies), with gradients G_i and momentum buffers M_i:
 *
 *   1. momentum          M <- beta * M + G
 *        ("Muon: The Orthogonalized Optimizer Explained Through Equations,
 *         Intuition, Code and Results", momentum recap note / Equation 1,
 *         plain-sum form);
 *   2. orthogonalize     O = NS_K(M): divide by ||M||_F + eps, then K times
 *                        A = X X^T, B = b A + c A A, X = a X + B X on the
 *                        wide side of the matrix
 *        (same page, Newton-Schulz section, Equation 6 and the code section);
 *        with tile_T > 0 the same map runs independently on every zero-padded
 *        tile_T x tile_T tile
 *        ("Hierarchical Muon: Tiled Newton-Schulz Updates for Efficient Muon
 *         Optimization", core claim and abstract);
 *   3. Hyperball         U_hat = O / ||O||_F, W <- rho * Pi(W - eta * U_hat),
 *                        Pi(x) = x / ||x||_F
 *        ("Fantastic Pretraining Optimizers and Where to Find Them II:
 *         Hyperball Optimization", §2 eq. 1 / Algorithm 1 and Method), where a
 *        numerically zero W - eta*U_hat restores the radius along the
 *        pre-update W instead of leaving zero ("Refactor of pre/post weight
 *        update hook functions", review comments on zero-norm handling);
 *      or RadialBrake    W' = W - eta * max(1, H/W)^0.5 * O, then
 *                        ||W_new|| = ||W|| + s (||W'|| - ||W||), s = outward
 *                        if the norm grew else inward
 *        (same hook page, PR description).
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers to caller-owned, contiguous,
 *     row-major buffers on the current HIP device.  The library never frees
 *     or retains them beyond the call.  Arrays of pointers, shapes, rho and
 *     coefficient tables are HOST memory, read during the call only.
 *   - Every argument is validated before any GPU work is queued: a call that
 *     returns MUONH_EINVAL, MUONH_ENOTIMPL or a planning MUONH_ENOMEM (the
 *     workspace of one matrix exceeds the limit) has changed nothing.  A
 *     failed allocation (MUONH_ENOMEM) also leaves the library's buffers as
 *     they were.  MUONH_EHIP means a HIP call failed; if it failed after
 *     some of the step's kernels were queued, those kernels still run, so
 *     params and moms may hold a partly applied step.
 *   - Work is queued asynchronously on opts->stream (NULL: the null stream).
 *     A call over two or more matrices that fit one workspace chunk runs
 *     some of them on library-owned side streams (opts->lanes), which start
 *     after earlier work on opts->stream and which opts->stream waits for
 *     before its next work: ordering is as if everything ran on
 *     opts->stream (opts->lanes = 1 keeps all work there).
 *   - Host synchronization: muonh_get_flags, muonh_reset_flags,
 *     muonh_profile_read and muonh_release synchronize.  A step, projection
 *     or orthogonalization never waits for the device, with two
 *     exceptions: the first call that needs a larger workspace (it frees
 *     the old one, which waits for the device), and allocation itself.  A
 *     call whose (buffers, shapes, options) are not in the plan cache builds
 *     its descriptor tables on the host and uploads them with the
 *     stream-ordered allocator and an asynchronous copy from pinned staging,
 *     both on opts->stream; the host does not wait for earlier work.  The
 *     cache holds the 32 most recently used call signatures; an evicted
 *     plan's tables are released in stream order.
 *   - Stream capture (HIP graphs): once a call with the same buffers, shapes
 *     and options has run eagerly, a repeat of it queues only kernels and
 *     event records / waits (no allocation, copy or memset) and can be
 *     captured, side streams included.  The graph holds addresses of the
 *     library's workspace and of that call's cached descriptor tables: it
 *     stays valid until the workspace grows, muonh_release runs, or 32
 *     other call signatures have pushed the call out of the plan cache.
 *     The reduction buffers a graph writes are never freed before
 *     muonh_release (a larger one replaces them without freeing them).
 *   - Determinism: every reduction is two-stage (one fp64 partial per block,
 *     then a fixed-order sum), so a call is bitwise reproducible for the same
 *     inputs, options and device, whatever opts->lanes and the chunking.
 *   - Zero norms are not errors: they follow the rules above and bump the
 *     device flag counters (muonh_get_flags).
 *   - Thread-compatible: calls from several host threads must not overlap.
 *     The library owns one workspace (grown on demand up to
 *     opts->workspace_limit, freed by muonh_release) and calls that share it
 *     are serialized on their streams by the caller.
 *   - Return value: MUONH_OK (0) or a negative MUONH_E* code; never throws.
 */
#ifndef MUONH_H
#define MUONH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MUONH_OK = 0,
  MUONH_EINVAL = -1,   /* invalid argument (null pointer, bad size, bad scalar, bad dtype) */
  MUONH_ENOMEM = -2,   /* workspace for one matrix exceeds workspace_limit, or allocation failed */
  MUONH_EHIP = -3,     /* a HIP runtime call or kernel launch failed */
  MUONH_ENOTIMPL = -4  /* valid request the library does not implement */
};

/* element types */
enum { MUONH_F32 = 0, MUONH_BF16 = 1 };

/* How Newton-Schulz with bf16 operands keeps X (and the Gram side) between
 * iterations; accumulation is fp32 in every mode:
 *   MUONH_NS_FOLD -- X itself is stored in bf16, as in the Muon explainer's
 *                    code section; a*X + B*X is formed in fp32 and rounded
 *                    once per iteration;
 *   MUONH_NS_X32  -- an fp32 master copy of X carries the a*X term, a bf16
 *                    shadow feeds the matrix cores (8 more bytes of traffic
 *                    per element and iteration);
 *   MUONH_NS_H16  -- the first iteration reads X0 and forms A0 = X0 X0^T and
 *                    B0 in bf16, as FOLD does; from X1 on, X, A and B are
 *                    stored in IEEE fp16 and the products after the first
 *                    iteration's run on fp16 operands (the matrix cores'
 *                    fp16 rate equals their bf16 rate).  Once the pre-scale
 *                    has been applied every iterate is bounded (singular
 *                    values below 1.25, |B| below 12), so fp16's range holds
 *                    them and its 3 more mantissa bits shrink the rounding
 *                    of X about 8x at FOLD's traffic (default).
 * All fold the 1/(||M||+eps) pre-scale into the first iteration instead of
 * rounding the pre-scaled X0, and when the NS input is not itself a bf16
 * value (fp32 state, or the Nesterov blend) all seed the first a*X0 term from
 * an fp32 copy of X0.  Resident tiles (tile sides <= 128) keep an fp32 master
 * X in registers under X32 and H16; tiles of side 129..256 on the fused
 * kernel hold X in bf16 under FOLD and H16.  Ignored when ns_dtype is
 * MUONH_F32. */
enum { MUONH_NS_FOLD = 0, MUONH_NS_X32 = 1, MUONH_NS_H16 = 2 };

/* weight-update hook */
enum { MUONH_HOOK_HYPERBALL = 0, MUONH_HOOK_RADIAL_BRAKE = 1, MUONH_HOOK_NONE = 2, MUONH_HOOK_RELATIVE = 3 };

/* Hyperball step length (opts.hyperball_step).  UNIT: W' = W - eta*U_hat, the
 * Hyperball show notes' Algorithm 1 (default).  RADIUS: W' = W - eta*rho*U_hat,
 * the hook PR description's wording (the update is normalized to the target
 * radius before it is applied).  Both then re-project onto radius rho. */
enum { MUONH_HB_STEP_UNIT = 0, MUONH_HB_STEP_RADIUS = 1 };

typedef struct muonh_opts {
  void*        stream;          /* hipStream_t to queue on; NULL = null stream */
  int          state_dtype;     /* dtype of grads, momentum, ns_orthogonalize in/out and
                                   frob_project's U: MUONH_BF16 (default) or MUONH_F32 */
  int          ns_dtype;        /* Newton-Schulz operand dtype: MUONH_BF16 (default) or MUONH_F32 */
  int          ns_precision;    /* MUONH_NS_H16 (default), MUONH_NS_FOLD or MUONH_NS_X32 */
  const float* coeffs;          /* host, 3*K floats: (a,b,c) for iteration k at [3k..3k+2];
                                   NULL = (3.4445, -4.7750, 2.0315) every iteration */
  float        ns_eps;          /* added to ||M||_F before dividing; default 1e-7 */
  float        zero_rel_eps;    /* Hyperball: ||W - eta*U_hat|| < zero_rel_eps*rho counts as
                                   zero and restores the radius; default 1e-6 */
  int          hook;            /* MUONH_HOOK_HYPERBALL (default), MUONH_HOOK_RADIAL_BRAKE,
                                   MUONH_HOOK_NONE (Muon's own update, see weight_decay) or
                                   MUONH_HOOK_RELATIVE (hook PR, review summary: the update is
                                   rescaled to the pre-update ||W||_F, W <- W - eta*||W||*O/||O||;
                                   O = 0 leaves W; no re-projection, rho ignored) */
  float        outward;         /* RadialBrake factor when the norm grows, in [0,1]; default 0.5 */
  float        inward;          /* RadialBrake factor otherwise, in [0,1]; default 1.0 */
  float        rb_eps;          /* RadialBrake: post-update norm <= rb_eps leaves W'; default 1e-15 */
  size_t       workspace_limit; /* bytes the library may hold as workspace; 0 = 3/4 of free HBM.
                                   Matrices are processed in chunks that fit it. */
  int          momentum_ema;    /* 0: M <- beta*M + G (default); 1: M <- beta*M + (1-beta)*G */
  int          nesterov;        /* 0: NS input is M (default); 1: the Nesterov blend,
                                   G + beta*M (sum form) or (1-beta)*G + beta*M (EMA form),
                                   formed from the updated M (Muon explainer, code section) */
  float        weight_decay;    /* MUONH_HOOK_NONE only: W <- W*(1 - eta*weight_decay) before
                                   the update (decoupled); finite, >= 0; default 0 */
  int          lanes;           /* concurrent lanes, 1..4; 0 = automatic: 2, but 1 when every
                                   matrix runs its Newton-Schulz as products of whole
                                   matrices or of tiles on the GEMM engine and one iteration
                                   over the set exceeds 2e12 flops (long products gain
                                   nothing from lanes), and 1 when every matrix runs on a
                                   resident-tile kernel (one launch per lane, nothing to fill).
                                   A call over
                                   two or more matrices that fit one workspace chunk is cut
                                   into that many runs of matrices, lane 0 on opts->stream and
                                   the others on library-owned side streams (see the stream
                                   convention above); 1: all work on opts->stream.  Results
                                   are identical for every value. */
  int          hyperball_step;  /* MUONH_HB_STEP_UNIT (default) or MUONH_HB_STEP_RADIUS; also
                                   used by frob_project */
  const int*   tile_sizes;      /* host, n entries, read during the call: per-matrix tile side
                                   for muonh_step / ns_orthogonalize (0: full-matrix NS; else
                                   the tile_T rules), overriding tile_T -- per-layer tile
                                   sizes (Hierarchical Muon page, discussion of tile choice
                                   by aspect ratio).  NULL (default): tile_T for every matrix */
  int          param_dtype;     /* dtype of params (master weights): MUONH_F32, the only one
                                   supported (anything else: MUONH_EINVAL) */
  int          deterministic;   /* 1 (default) or 0.  Every reduction is two-stage and bitwise
                                   reproducible either way; 0 selects no faster path */
} muonh_opts;

/* Fill *o with the defaults listed above. */
void muonh_default_opts(muonh_opts* o);

/*
 * muonh_step -- one full optimizer step (momentum -> NS -> hook) for n matrices.
 * With MUONH_HOOK_NONE the update is Muon's own (Muon explainer, code
 * section): W <- W*(1 - eta*weight_decay) - eta*max(1, H/W)^0.5 * O.
 *
 *   params[i]  device, fp32, shapes[2i] x shapes[2i+1], updated in place (W)
 *   grads[i]   device, state_dtype, same shape, read only (G)
 *   moms[i]    device, state_dtype, same shape, updated in place (M)
 *   shapes     host, 2*n int64: rows, cols of matrix i (each >= 1; with
 *              tile_T = 0 or > 128, (pad256(longer side) * pad64(shorter
 *              side) + 256) * operand bytes must stay below 4 GiB, else
 *              MUONH_ENOTIMPL)
 *   n          number of matrices (>= 1)
 *   eta        learning rate / Hyperball angular step (finite, >= 0)
 *   beta       momentum coefficient, in [0, 1)
 *   K          Newton-Schulz iterations, 0..64 (0: O = M / (||M|| + eps))
 *   rho        host, n floats: Hyperball radius per matrix (finite, > 0);
 *              ignored (may be NULL) for RadialBrake, MUONH_HOOK_NONE and
 *              MUONH_HOOK_RELATIVE
 *   tile_T     0 = full-matrix NS; > 0 = Hierarchical Muon with tile side tile_T
 *              (1..128, or a multiple of 64 up to 8192); the hook always acts on
 *              the full matrix
 *   opts       NULL = defaults
 * Buffers of different matrices must not overlap; grads may not alias moms.
 */
int muonh_step(void* const params[], const void* const grads[], void* const moms[],
               const int64_t shapes[], int n, float eta, float beta, int K,
               const float rho[], int tile_T, const muonh_opts* opts);

/*
 * muonh_step_noalloc -- muonh_step for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, options and results as muonh_step (the
 * same kernels; bitwise the same output), but the call allocates nothing:
 * its workspace, descriptor tables and reduction partials live in a static
 * device array of MUONH_NOALLOC_SCRATCH_BYTES per GPU, which each GPU the
 * library runs on holds until the process ends.
 *   - Limit: the call's workspace may use 3/4 of the scratch (48 MiB), the
 *     rest holds its tables and partials.  A call that needs more returns
 *     MUONH_ENOMEM before queuing any work, and muonh_last_error() names the
 *     sizes.  (Resident tiles, tile_T <= 128, need only the bf16 O buffer of
 *     each matrix: 2 bytes per element; full-matrix Newton-Schulz needs the
 *     X ping-pong, A, B and O buffers, about 13 MB for a 768 x 2304 matrix.)
 *   - Every call on a GPU uses that GPU's one scratch and keeps the last
 *     call's contents: calls queued on one stream are ordered, but calls that
 *     overlap on one GPU (other streams, other threads, no ordering between
 *     them) race and corrupt each other's results.
 *   - All work is queued on opts->stream (opts->lanes is ignored: one lane).
 *     Nothing is cached: each call plans on the host and uploads its tables
 *     with one stream-ordered copy from host memory.
 */
#define MUONH_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int muonh_step_noalloc(void* const params[], const void* const grads[], void* const moms[],
                       const int64_t shapes[], int n, float eta, float beta, int K, const float rho[],
                       int tile_T, const muonh_opts* opts);

/*
 * adamh_step -- AdamH: the Hyperball wrapper around Adam's update (Hyperball
 * show notes, Method: any base step, Adam's preconditioned update first
 * among them; Key claims and Results report AdamH).  Adam itself (Muon
 * explainer, Equation 2 and its text; the bias-corrected form of the Adam
 * paper the Hyperball page cites):
 *   m <- beta1*m + (1-beta1)*g,   v <- beta2*v + (1-beta2)*g^2,
 *   U  = (m / (1-beta1^step)) / (sqrt(v / (1-beta2^step)) + eps)
 * then opts->hook acts on U as on Muon's O, without Muon's shape scale:
 * Hyperball (default; opts->hyperball_step honored), RadialBrake,
 * MUONH_HOOK_RELATIVE, or MUONH_HOOK_NONE = plain AdamW,
 * W <- W*(1 - eta*weight_decay) - eta*U.
 *
 *   params[i]      device, fp32, updated in place (W)
 *   grads[i]       device, opts->state_dtype, read only (g)
 *   exp_avg[i]     device, fp32, updated in place (m)
 *   exp_avg_sq[i]  device, fp32, updated in place (v)
 *   shapes         host, 2*n int64 rows, cols (each >= 1)
 *   eta            learning rate (finite, >= 0)
 *   beta1, beta2   in [0, 1); eps finite > 0 (1e-8 is Adam's usual value)
 *   step           1-based count of this step (bias corrections), >= 1
 *   rho            host, n floats, Hyperball radius (finite, > 0); ignored
 *                  (may be NULL) for the other hooks
 * Two streaming passes: moments + the hook's norms (||U||^2, <W,U>,
 * ||W||^2; ||W - c U||^2 is formed from them), then the hook.  U is
 * recomputed in pass 2 from the stored moments, never stored.
 * Buffers of different matrices must not overlap; grads, exp_avg and
 * exp_avg_sq of one matrix must be distinct.
 */
int adamh_step(void* const params[], const void* const grads[], void* const exp_avg[],
               void* const exp_avg_sq[], const int64_t shapes[], int n, float eta, float beta1,
               float beta2, float eps, int64_t step, const float rho[], const muonh_opts* opts);

/*
 * ns_orthogonalize -- out[i] = NS_K(in[i]), no momentum, no hook: the
 * Newton-Schulz map of the Muon explainer (Newton-Schulz section, Equation 6,
 * and the code section's newton_schulz5: divide by ||X||_F + eps, then K
 * times A = X X^T, B = b A + c A A, X = a X + B X on the wide side); with
 * tile_T > 0 the same map on every zero-padded tile_T x tile_T tile
 * (Hierarchical Muon page, core claim and abstract).
 *   in[i]   device, opts->state_dtype, shapes[2i] x shapes[2i+1], read only
 *   out[i]  device, same dtype and shape, written; may alias in[i]
 * Same shape, K, tile_T and opts rules (and errors) as muonh_step; a zero
 * input gives a zero output (the eps).
 */
int ns_orthogonalize(const void* const in[], void* const out[], const int64_t shapes[],
                     int n, int K, int tile_T, const muonh_opts* opts);

/*
 * frob_project -- the Hyperball projection on its own (Hyperball show notes,
 * §2 eq. 1 / Algorithm 1 and Method: U_hat = U / ||U||_F,
 * W <- rho * Pi(W - eta * U_hat), Pi(x) = x / ||x||_F):
 *   W[i] <- rho[i] * Pi(W[i] - eta * U[i] / ||U[i]||)
 * (eta * rho[i] * U[i] / ||U[i]|| with opts->hyperball_step = RADIUS)
 * with the same zero rules as muonh_step (zero U: projection only; a
 * numerically zero W' restores the radius along W; W = 0 is left and
 * counted).
 *   W[i]    device, fp32, shapes[2i] x shapes[2i+1], updated in place
 *   U       NULL (plain projection W <- rho * W / ||W||) or an array of n
 *           device buffers of opts->state_dtype, same shapes, read only (a
 *           NULL entry is a zero update)
 *   eta     finite, >= 0;  rho  host, n floats, finite, > 0
 * Errors as muonh_step (MUONH_EINVAL for a bad pointer, shape or scalar).
 */
int frob_project(void* const W[], const void* const U[], const int64_t shapes[], int n,
                 float eta, const float rho[], const muonh_opts* opts);

/*
 * Device flag counters, accumulated since the last reset:
 *   out[0] matrices whose orthogonalized update had zero norm,
 *   out[1] Hyperball radius restores (numerically zero post-update weight),
 *   out[2] restores impossible because W was zero too (W left unchanged),
 *   out[3] matrices with a non-finite norm.
 * Synchronizes the device.  Returns MUONH_OK or MUONH_EHIP.
 */
int muonh_get_flags(uint64_t out[4]);
int muonh_reset_flags(void);

/* Static message for an error code. */
const char* muonh_strerror(int code);

/* Free the workspace and cached plans (synchronizes the device first). */
void muonh_release(void);

/*
 * Host-only planning query (no GPU call): how a muonh_step with these
 * arguments would be split.  out[0] = chunks run one after another,
 * out[1] = workspace bytes the call needs (the largest chunk; when the set
 * fits in one chunk and holds two or more matrices, the sum over the lanes
 * that run side by side), out[2] = Newton-Schulz units (matrices or tiles),
 * out[3] = dense NS flops per step (sum of K (4 r^2 s + 2 r^3) over units,
 * with r, s the true (unpadded) sides), out[4] = GEMM tile jobs per NS
 * iteration, out[5] = streaming bytes per step (momentum 3 passes + hook
 * 2 passes, algorithmic), out[6] = concurrent lanes.  Returns MUONH_OK,
 * MUONH_EINVAL or MUONH_ENOMEM exactly as muonh_step's validation would.
 */
int muonh_plan_query(const int64_t shapes[], int n, int K, int tile_T,
                     const muonh_opts* opts, size_t workspace_limit, int64_t out[7]);

/*
 * Per-kernel timing for measurement.  muonh_profile_begin() makes every later
 * launch record a pair of HIP events on the stream it is queued on;
 * muonh_profile_read() synchronizes, and fills up to max entries with the
 * accumulated launch count, total milliseconds and algorithmic work of each
 * kernel class since begin (flops for Newton-Schulz kernels, bytes for
 * streaming kernels), then stops recording.  *n_out receives the entry count.
 */
typedef struct muonh_kernel_stat {
  char     name[40];
  uint64_t launches;
  double   total_ms;
  double   flops;   /* algorithmic flops over all recorded launches */
  double   bytes;   /* algorithmic HBM bytes over all recorded launches */
} muonh_kernel_stat;

int muonh_profile_begin(void);
int muonh_profile_read(muonh_kernel_stat* out, int max, int* n_out);

/* Library version string. */
const char* muonh_version(void);

/* Text of the last HIP failure behind a MUONH_EHIP return on this host
 * thread (the failing call and HIP's error string), or of the sizes behind a
 * muonh_step_noalloc MUONH_ENOMEM ("" if none). */
const char* muonh_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MUONH_H */
