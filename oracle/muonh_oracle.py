"""Plain fp64 CPU oracle for the MuonH / Hierarchical-Muon optimizer step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers or constants); its inputs come from the
seeded generators in ``synth/`` or from the tests themselves.

Everything is computed in float64 with numpy, step by step in the order the
pages give, with no blocking, fusion or reordering.  Sources (page titles):

* [MUON]  "Muon: The Orthogonalized Optimizer Explained Through Equations,
  Intuition, Code and Results" -- momentum recap note and Equation 1 (the
  momentum buffer), the Newton-Schulz section with Equation 6 (odd quintic
  p(s) = a s + b s^3 + c s^5 acting on singular values; Frobenius pre-scale),
  and the code section (``newton_schulz5``: bf16 cast, wide-side Gram,
  eps = 1e-7, (a, b, c) = (3.4445, -4.7750, 2.0315), transpose back).
* [HB]    "Fantastic Pretraining Optimizers and Where to Find Them II:
  Hyperball Optimization" -- TL;DR, Key claims (§2 eq. 1, Algorithm 1) and the
  Method section: U_hat = U / ||U||_F, W <- rho * Pi(W - eta * U_hat),
  Pi(x) = x / ||x||_F, rho = ||W_0||_F.
* [HOOKS] "Refactor of pre/post weight update hook functions" (NVIDIA-NeMo
  Emerging-Optimizers PR #224) -- the PR description (RadialBrake norm rule,
  the pre/post hook order) and the review comments (zero-norm handling must
  restore the radius instead of leaving zero; eps-based zero tests; RadialBrake
  eps default 1e-15; no amplifying scale factors).
* [HIMUON] "Hierarchical Muon: Tiled Newton-Schulz Updates for Efficient Muon
  Optimization" -- core claim and abstract: cut each momentum matrix into
  T x T tiles, apply the same finite Newton-Schulz map to every tile
  independently, reassemble.
* [NMUON] "The Newton-Muon Optimizer" -- abstract: msgn(X) = U V^T for a
  compact SVD X = U S V^T (used only as a sanity band, never as the target).
* Adam (for AdamH): [MUON] Equation 2 and its text (two running averages,
  the gradient's divided by the square root of the squared gradient's); the
  equation itself did not survive extraction, so the bias-corrected form of
  the Adam paper on [HB]'s reference list is taken, with the betas of the
  [MUON] code section's AdamW (0.9, 0.95) as defaults and eps = 1e-8.

Readings taken where the pages are silent:

* momentum is the plain sum M <- beta*M + G, no Nesterov blend, unless asked
  for: the exponential-average buffer and the Nesterov blend follow [MUON]
  code section (``lerp_`` forms); with the plain sum the blend is G + beta*M;
* the NS eps is added to the Frobenius norm (not a max);
* a matrix is transposed iff it has more rows than columns (square: not);
* a HiMuon tile is zero-padded to T x T, gets its own pre-scale, and the grid
  is anchored at (0, 0);
* Hyperball: if ||W - eta*U_hat|| < zero_rel_eps * rho the post-update weight
  counts as numerically zero and the radius is restored along the pre-update
  W; if W is zero as well it is left unchanged and flagged;
* RadialBrake: the update is Muon's O with the shape scale max(1, H/W)^0.5;
  outward when the norm strictly grows; a post-update norm <= eps leaves W';
* RelativeUpdate: the update is rescaled to the pre-update ||W||_F (no
  post-update step); the Hyperball hook's "normalize to the target radius"
  wording is the optional radius-sized step, the unit step stays the default.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(closed forms, the pages' worked examples, invariants, brute force on tiny
inputs).  The pages' RadialBrake test targets 7.5 / 9.0 come without their
inputs: beyond the formula itself that part is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

# Newton-Schulz quintic coefficients tuned for a steep slope at zero
# ([MUON] Newton-Schulz section and code section).
KELLER_ABC = (3.4445, -4.7750, 2.0315)
# eps added to the Frobenius norm before dividing ([MUON] code section).
NS_EPS = 1e-7
# RadialBrake's default eps for "numerically zero" norms ([HOOKS] review).
RB_EPS = 1e-15

FLAG_PROJECTED = "projected"
FLAG_RESTORED = "restored"
FLAG_UNRESTORABLE = "unrestorable"


def _f64(x) -> np.ndarray:
    return np.array(x, dtype=np.float64, copy=True)


def round_to_bf16(x) -> np.ndarray:
    """Emulate storage of ``x`` in a bfloat16 tensor: round-to-nearest-even to
    8 significant bits, returned as float64 values.

    This is the storage format a bf16 momentum buffer imposes (the workload
    keeps momentum in bf16); it is not part of the pages' arithmetic.
    """
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32).astype(np.float64)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = np.nan
    return out


# ---------------------------------------------------------------------------
# a1: momentum
# ---------------------------------------------------------------------------
def momentum_update(M, G, beta) -> np.ndarray:
    """M <- beta * M + G.

    [MUON] momentum recap note / Equation 1: SGD momentum keeps a running sum
    of gradients with coefficient mu; the write-up's Equation 1 uses the plain
    sum (no (1 - mu) factor), which is the form taken here.
    """
    return float(beta) * _f64(M) + _f64(G)


def momentum_update_ema(M, G, beta) -> np.ndarray:
    """The exponential-average form of the same buffer, beta*M + (1-beta)*G,
    as in [MUON] code section (the buffer is lerped toward the gradient by
    1 - mu)."""
    b = float(beta)
    return b * _f64(M) + (1.0 - b) * _f64(G)


def nesterov_input(G, M_new, beta, ema: bool) -> np.ndarray:
    """The Newton-Schulz input of a Nesterov step, from the fresh gradient and
    the already-updated buffer.

    [MUON] code section: the update is the gradient lerped toward the buffer
    by mu, (1 - mu) G + mu M.  For the plain-sum buffer of Equation 1 (which
    carries no (1 - mu) factor on G) the same look-ahead is G + mu M.
    """
    b = float(beta)
    if ema:
        return (1.0 - b) * _f64(G) + b * _f64(M_new)
    return _f64(G) + b * _f64(M_new)


# ---------------------------------------------------------------------------
# a2-a6: Newton-Schulz orthogonalization
# ---------------------------------------------------------------------------
def _coeff_list(K, coeffs):
    if coeffs is None:
        return [KELLER_ABC] * K
    c = [tuple(float(v) for v in row) for row in coeffs]
    if len(c) < K:
        raise ValueError("coefficient table shorter than K")
    return c[:K]


def newton_schulz(G, K: int = 5, coeffs=None, eps: float = NS_EPS) -> np.ndarray:
    """K quintic Newton-Schulz steps on the wide side of ``G``.

    [MUON] Newton-Schulz section, Equation 6 and code section:
      1. work on the transpose if the matrix is tall, so the Gram X X^T is
         the small (r x r) one;
      2. divide by the Frobenius norm plus eps, which puts every singular
         value in (0, 1];
      3. repeat K times: A = X X^T; B = b A + c A A; X = a X + B X
         (this is a X + b (X X^T) X + c (X X^T)^2 X);
      4. transpose back.
    ``coeffs`` optionally gives one (a, b, c) row per iteration.
    """
    X = _f64(G)
    if X.ndim != 2:
        raise ValueError("newton_schulz expects a matrix")
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.T
    X = X / (np.linalg.norm(X) + eps)
    for a, b, c in _coeff_list(K, coeffs):
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    if tall:
        X = X.T
    return np.ascontiguousarray(X)


def tiled_newton_schulz(M, T: int, K: int = 5, coeffs=None, eps: float = NS_EPS) -> np.ndarray:
    """Hierarchical Muon: the same finite NS map on every T x T tile.

    [HIMUON] core claim / abstract: partition the H x W matrix into T x T
    tiles, apply the NS map to each tile on its own, reassemble.  Readings:
    the grid starts at (0, 0); an edge tile that does not fill T x T is
    zero-padded to T x T before the map and cropped after it; each tile is
    pre-scaled by its own Frobenius norm, since every tile runs the
    identical map.
    """
    X = _f64(M)
    H, W = X.shape
    if T <= 0:
        raise ValueError("tile side must be positive")
    out = np.zeros_like(X)
    for r0 in range(0, H, T):
        for c0 in range(0, W, T):
            blk = X[r0:r0 + T, c0:c0 + T]
            h, w = blk.shape
            tile = np.zeros((T, T), dtype=np.float64)
            tile[:h, :w] = blk
            o = newton_schulz(tile, K, coeffs, eps)
            out[r0:r0 + h, c0:c0 + w] = o[:h, :w]
    return out


def orthogonalize(M, K: int = 5, tile_T: int = 0, coeffs=None, eps: float = NS_EPS) -> np.ndarray:
    """Full-matrix NS when tile_T == 0, tiled (HiMuon) NS otherwise."""
    if tile_T and tile_T > 0:
        return tiled_newton_schulz(M, tile_T, K, coeffs, eps)
    return newton_schulz(M, K, coeffs, eps)


def msgn_svd(X) -> np.ndarray:
    """msgn(X) = U V^T from a compact SVD ([NMUON] abstract; [MUON] update
    rule section).  A sanity band for NS, not what NS computes."""
    U, _, Vt = np.linalg.svd(_f64(X), full_matrices=False)
    return U @ Vt


# ---------------------------------------------------------------------------
# a8-a10: Hyperball
# ---------------------------------------------------------------------------
def hyperball(W, U, eta, rho, zero_rel_eps: float = 1e-6, step: str = "unit"):
    """One Hyperball update of W with base-optimizer direction U.

    [HB] Method / §2 eq. 1, Algorithm 1:
      U_hat = U / ||U||_F              (unit Frobenius direction)
      W'    = W - eta * U_hat
      W     <- rho * W' / ||W'||_F     (re-project onto the sphere of radius rho)
    ``step="radius"`` takes the [HOOKS] PR description's wording instead (the
    Hyperball hook normalizes the update to the target radius before the
    update): W' = W - eta * rho * U_hat.
    Zero handling ([HOOKS] review: an exactly cancelling update must restore
    the radius rather than leave zero; numerical zero is tested against an
    eps, not with == 0):
      * ||U|| == 0            -> U_hat = 0 (only the projection happens);
      * ||W'|| < eps*rho      -> restore: W <- rho * W / ||W||;
      * ... and ||W|| == 0    -> W unchanged, flagged.
    Returns (W_new, flag).
    """
    W = _f64(W)
    U = _f64(U)
    rho = float(rho)
    eta = float(eta)
    if step not in ("unit", "radius"):
        raise ValueError("step must be 'unit' or 'radius'")
    nU = np.linalg.norm(U)
    U_hat = U / nU if nU > 0 else np.zeros_like(U)
    Wp = W - (eta * rho if step == "radius" else eta) * U_hat
    n = np.linalg.norm(Wp)
    if n >= zero_rel_eps * rho:
        return rho * Wp / n, FLAG_PROJECTED
    nW = np.linalg.norm(W)
    if nW > 0:
        return rho * W / nW, FLAG_RESTORED
    return W, FLAG_UNRESTORABLE


def shape_scale(H: int, W: int) -> float:
    """max(1, H/W)^0.5 -- the shape scaling of Muon's O ([MUON] code section,
    Muon class)."""
    return max(1.0, H / W) ** 0.5


def radial_brake(W, O, eta, outward: float = 0.5, inward: float = 1.0, eps: float = RB_EPS):
    """RadialBrake hook around a plain Muon update.

    [HOOKS] PR description: take the optimizer's usual update
    w = w_prev - eta * O' (O' = shape-scaled Muon direction), then rescale w so
    that ||w_brake|| = ||w_prev|| + s (||w|| - ||w_prev||), with s = outward
    when the norm grew and s = inward otherwise.  A post-update norm at or
    below eps leaves w as is.  Returns the new W.
    """
    W = _f64(W)
    O = _f64(O)
    H, Wd = W.shape
    Wp = W - float(eta) * shape_scale(H, Wd) * O
    n0 = np.linalg.norm(W)
    n1 = np.linalg.norm(Wp)
    s = float(outward) if n1 > n0 else float(inward)
    if n1 > eps:
        return Wp * ((n0 + s * (n1 - n0)) / n1)
    return Wp


def plain_update(W, O, eta, weight_decay: float = 0.0):
    """Muon's own weight update with no hook ([MUON] code section, ``step``):
    decoupled weight decay W <- W (1 - eta * wd), then W <- W - eta * O'
    with the shape-scaled direction O' = max(1, H/W)^0.5 O."""
    W = _f64(W)
    H, Wd = W.shape
    W = W * (1.0 - float(eta) * float(weight_decay))
    return W - float(eta) * shape_scale(H, Wd) * _f64(O)


def relative_update(W, O, eta):
    """RelativeUpdate hook ([HOOKS] review summary, file table: the pre-update
    scaling matches the update's norm to the current weight norm): the update
    O is rescaled to ||O'||_F = ||W||_F, then W <- W - eta * O', i.e.
    W - eta * ||W||_F * O / ||O||_F.  A zero O leaves W unchanged.  (The shape
    scale of Muon's O cancels in the rescaling.)"""
    W = _f64(W)
    O = _f64(O)
    nO = np.linalg.norm(O)
    if not nO > 0:
        return W.copy()
    return W - float(eta) * (np.linalg.norm(W) / nO) * O


# ---------------------------------------------------------------------------
# frob_project and the whole step
# ---------------------------------------------------------------------------
def frob_project(W, U, eta, rho, zero_rel_eps: float = 1e-6, step: str = "unit"):
    """W <- rho * Pi(W - eta * U/||U||) (``step="radius"``: eta * rho * U/||U||);
    ``U is None`` is the plain projection W <- rho * W / ||W|| ([HB] Method)."""
    if U is None:
        U = np.zeros_like(_f64(W))
    return hyperball(W, U, eta, rho, zero_rel_eps, step)


def muonh_step(Ws, Gs, Ms, eta, beta, K, rhos, tile_T: int = 0, hook: str = "hyperball",
               coeffs=None, outward: float = 0.5, inward: float = 1.0,
               zero_rel_eps: float = 1e-6, state_bf16: bool = False,
               ema: bool = False, nesterov: bool = False, weight_decay: float = 0.0,
               hb_step: str = "unit", tile_sizes=None):
    """One MuonH (or HiMuon-H / Muon+RadialBrake / plain Muon) step over a
    list of matrices.

    Per matrix, in the pages' order: momentum ([MUON] Eq. 1, or the
    exponential average of the code section with ``ema``) -> the Newton-Schulz
    input (the buffer, or the Nesterov blend with ``nesterov``) -> NS ([MUON]
    Eq. 6 / code; tiled per [HIMUON] when tile_T > 0) -> Hyperball ([HB]
    Algorithm 1; ``hb_step`` selects the unit or radius-sized step),
    RadialBrake ([HOOKS]), RelativeUpdate (``"relative"``, [HOOKS]) or no hook
    (``"none"``: Muon's own update with decoupled weight decay).

    ``state_bf16`` models a bf16 momentum buffer: the updated M is stored
    rounded to bf16 and the NS input is formed from the stored value.
    ``tile_sizes`` gives each matrix its own tile side (0: full matrix;
    [HIMUON] discussion: tile sizes chosen per layer).

    Returns (new_Ws, new_Ms, Os, flags).
    """
    new_W, new_M, Os, flags = [], [], [], []
    for i, (W, G, M) in enumerate(zip(Ws, Gs, Ms)):
        m = momentum_update_ema(M, G, beta) if ema else momentum_update(M, G, beta)
        if state_bf16:
            m = round_to_bf16(m)
        x = nesterov_input(G, m, beta, ema) if nesterov else m
        O = orthogonalize(x, K, tile_T if tile_sizes is None else tile_sizes[i], coeffs)
        if hook == "hyperball":
            w, f = hyperball(W, O, eta, rhos[i], zero_rel_eps, hb_step)
        elif hook == "relative":
            w, f = relative_update(W, O, eta), None
        elif hook == "radial_brake":
            w, f = radial_brake(W, O, eta, outward, inward), None
        elif hook == "none":
            w, f = plain_update(W, O, eta, weight_decay), None
        else:
            raise ValueError("unknown hook")
        new_W.append(w)
        new_M.append(m)
        Os.append(O)
        flags.append(f)
    return new_W, new_M, Os, flags


# ---------------------------------------------------------------------------
# AdamH: Hyperball around Adam's preconditioned update
# ---------------------------------------------------------------------------
def adam_direction(M, V, G, beta1, beta2, eps, t):
    """Adam's per-coordinate update direction ([MUON] Equation 2 and the text
    around it: a running average of the gradient and one of its square, the
    first divided by the square root of the second; the Adam paper cited on
    the Hyperball page's reference list adds the bias corrections):
      m <- beta1 m + (1 - beta1) g,   v <- beta2 v + (1 - beta2) g^2,
      U  = (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps).
    Returns (m, v, U) in float64; t >= 1 counts this step."""
    M, V, G = _f64(M), _f64(V), _f64(G)
    b1, b2, t = float(beta1), float(beta2), int(t)
    m = b1 * M + (1.0 - b1) * G
    v = b2 * V + (1.0 - b2) * G * G
    U = (m / (1.0 - b1 ** t)) / (np.sqrt(v / (1.0 - b2 ** t)) + float(eps))
    return m, v, U


def adamh_step(Ws, Gs, Ms, Vs, eta, beta1, beta2, eps, t, rhos=None, hook: str = "hyperball",
               outward: float = 0.5, inward: float = 1.0, zero_rel_eps: float = 1e-6,
               weight_decay: float = 0.0, hb_step: str = "unit", state_f32: bool = True):
    """AdamH ([HB] Method: Hyperball wraps any base optimizer step, Adam's
    preconditioned update named first; Key claims and Results report AdamH).
    Per matrix: Adam's direction U (``adam_direction``), then the hook:
    Hyperball (default), RadialBrake, RelativeUpdate, or ``"none"`` -- plain
    AdamW, W <- W (1 - eta wd) - eta U.  There is no shape scale (that is
    Muon's).  ``state_f32`` models fp32 storage of m and v: U is formed from
    the stored (fp32-rounded) moments.  Returns (new_Ws, new_Ms, new_Vs, Us, flags)."""
    out_w, out_m, out_v, Us, flags = [], [], [], [], []
    for i, (W, G, M, V) in enumerate(zip(Ws, Gs, Ms, Vs)):
        m, v, U = adam_direction(M, V, G, beta1, beta2, eps, t)
        if state_f32:
            m = m.astype(np.float32).astype(np.float64)
            v = v.astype(np.float32).astype(np.float64)
            b1, b2 = float(beta1), float(beta2)
            U = (m / (1.0 - b1 ** int(t))) / (np.sqrt(v / (1.0 - b2 ** int(t))) + float(eps))
        Wd = _f64(W)
        if hook == "hyperball":
            w, f = hyperball(Wd, U, eta, rhos[i], zero_rel_eps, hb_step)
        elif hook == "relative":
            w, f = relative_update(Wd, U, eta), None
        elif hook == "radial_brake":
            Wp = Wd - float(eta) * U
            n0, n1 = np.linalg.norm(Wd), np.linalg.norm(Wp)
            s = float(outward) if n1 > n0 else float(inward)
            w, f = (Wp * ((n0 + s * (n1 - n0)) / n1) if n1 > RB_EPS else Wp), None
        elif hook == "none":
            w, f = Wd * (1.0 - float(eta) * float(weight_decay)) - float(eta) * U, None
        else:
            raise ValueError("unknown hook")
        out_w.append(w)
        out_m.append(m)
        out_v.append(v)
        Us.append(U)
        flags.append(f)
    return out_w, out_m, out_v, Us, flags
