"""Pins for the fp64 oracle: it is checked against what the pages and the
mathematics fix, never against itself.

* closed form of an odd matrix polynomial (the Muon explainer's Newton-Schulz
  section: directions pass through, each singular value goes through the
  scalar polynomial);
* the worked examples the Muon explainer prints (tests/golden);
* special cases that reduce to textbook results (Newton-Schulz polar
  iteration, 1x1 matrices, orthogonal inputs) and to an SVD band;
* Hyperball and RadialBrake closed forms and invariants (Hyperball show notes,
  hook PR);
* HiMuon identities (tile >= matrix, 1x1 tiles, locality, zero padding);
* a few planted mistakes to show that the pins catch them.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import muonh_oracle as orc
from synth import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
ABC = (3.4445, -4.7750, 2.0315)


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


EX = {c["id"]: c for c in _load("muon_explainer_worked_examples.json")["cases"]}
HB = _load("hyperball_hooks_examples.json")


def scalar_iterate(x, K, abc=ABC):
    """K applications of the scalar quintic a x + b x^3 + c x^5 (elementwise)."""
    x = np.asarray(x, dtype=np.float64)
    a, b, c = abc
    for _ in range(K):
        x = a * x + b * x ** 3 + c * x ** 5
    return x


def sv(X):
    return np.linalg.svd(X, compute_uv=False)


# ---------------------------------------------------------------------------
# closed form: NS(U diag(s) V^T) = U diag(p^K(s / (||s|| + eps))) V^T
# ---------------------------------------------------------------------------

def closed_form_error(ns_fn, H, W, K, seed):
    k = min(H, W)
    s = np.linspace(1.0, 0.02, k) * 3.7  # arbitrary scale: the pre-scale removes it
    U = gen.orthonormal(H, k, seed)
    V = gen.orthonormal(W, k, seed + 7)
    X = (U * s) @ V.T
    sn = s / (np.linalg.norm(s) + 1e-7)
    expect = (U * scalar_iterate(sn, K)) @ V.T
    got = ns_fn(X, K)
    if got.shape != expect.shape:
        return np.inf
    return np.linalg.norm(got - expect) / np.linalg.norm(expect)


@pytest.mark.parametrize("H,W", [(5, 7), (7, 5), (6, 6), (33, 17), (17, 33), (1, 9), (9, 1), (64, 128)])
@pytest.mark.parametrize("K", [0, 1, 2, 5])
def test_ns_closed_form(H, W, K):
    err = closed_form_error(lambda X, K: orc.newton_schulz(X, K), H, W, K, seed=H * 100 + W)
    assert err < 1e-12


def test_ns_closed_form_rank_deficient():
    # Rank-2 10x14: the zero singular values stay zero (p is odd, p(0) = 0).
    U = gen.orthonormal(10, 2, 3)
    V = gen.orthonormal(14, 2, 4)
    s = np.array([2.0, 0.5])
    X = (U * s) @ V.T
    got = orc.newton_schulz(X, 5)
    expect = (U * scalar_iterate(s / (np.linalg.norm(s) + 1e-7), 5)) @ V.T
    assert np.linalg.norm(got - expect) < 1e-12
    assert np.sum(sv(got) > 1e-10) == 2


def test_ns_per_iteration_coefficient_table():
    # A coefficient table applies row k at iteration k (DeepSeek-V4 two-stage).
    U = gen.orthonormal(12, 12, 11)
    V = gen.orthonormal(12, 12, 12)
    s = np.geomspace(1.0, 0.01, 12)
    X = (U * s) @ V.T
    table = [ABC] * 8 + [(2.0, -1.5, 0.5)] * 2
    x = s / (np.linalg.norm(s) + 1e-7)
    for row in table:
        x = scalar_iterate(x, 1, row)
    got = orc.newton_schulz(X, 10, coeffs=table)
    assert np.linalg.norm(got - (U * x) @ V.T) < 1e-12


# ---------------------------------------------------------------------------
# worked examples printed on the Muon explainer page
# ---------------------------------------------------------------------------

def _diag_embed(s, seed):
    n = len(s)
    return gen.with_singular_values(n, n, s, seed)


def test_worked_two_by_two():
    c = EX["two_by_two_ellipse"]
    out = np.sort(sv(orc.newton_schulz(_diag_embed(c["sigma_in"], 1), c["K"])))
    # singular values come out sorted; the page lists (rare -> 0.75, dominant -> 0.70)
    assert np.allclose(np.round(out, c["decimals"]), sorted(c["sigma_out"]))


def test_worked_five_directions():
    c = EX["five_directions"]
    s = np.array(c["sigma_in"])
    assert round(float(np.linalg.norm(s)), c["frobenius_norm_decimals"]) == c["frobenius_norm"]
    pre = s / (np.linalg.norm(s) + 1e-7)
    for v, p, d in zip(pre, c["prescaled"], c["prescaled_decimals"]):
        assert round(float(v), d) == p
    out = sv(orc.newton_schulz(_diag_embed(s, 2), c["K"]))
    assert round(float(out.min()), c["decimals"]) == c["sigma_out_min"]
    assert round(float(out.max()), c["decimals"]) == c["sigma_out_max"]
    assert round(float(s.max() / s.min())) == c["condition_in"]
    assert round(float(out.max() / out.min()), c["condition_out_decimals"]) == c["condition_out"]


def test_worked_textbook_cubic():
    c = EX["textbook_cubic"]
    # A 2x2 whose pre-scaled singular values are (sqrt(1 - 0.01^2), 0.01).
    t = c["sigma_prescaled"]
    s = np.array([math.sqrt(1 - t * t), t]) * (1 + 1e-7)
    out = sv(orc.newton_schulz(_diag_embed(s, 5), c["K"], coeffs=[c["coeffs"]] * c["K"]))
    assert round(float(out.min()), c["decimals"]) == c["sigma_out"]


def test_worked_slope_at_zero():
    # d/ds of NS at a vanishing singular value, one step: a (numerically, from
    # a matrix whose smallest pre-scaled singular value is tiny).
    s = np.array([1.0, 1e-9])
    X = _diag_embed(s, 6)
    out = sv(orc.newton_schulz(X, 1))
    pre_small = 1e-9 / (np.linalg.norm(s) + 1e-7)
    assert abs(out.min() / pre_small - EX["slope_at_zero"]["slope"]) < 1e-6


def test_worked_band_after_five_steps():
    c = EX["band_after_five_steps"]
    lo, hi = c["sigma_prescaled_range"]
    # Matrices whose pre-scaled singular values span [0.01, ~1): one dominant
    # direction near 1, the rest spread down to 0.01.
    outs = []
    for seed in range(6):
        r = gen.rng(seed).uniform(lo, 0.12, size=15)
        s = np.concatenate([[1.0], r, [lo]])
        s[0] = math.sqrt(max(1.0 - float(np.sum(s[1:] ** 2)), 0.5))
        X = _diag_embed(s, 40 + seed)
        pre = s / (np.linalg.norm(s) + 1e-7)
        assert pre.min() >= lo * 0.999 and pre.max() <= hi
        outs.append(sv(orc.newton_schulz(X, c["K"])))
    allv = np.concatenate(outs)
    assert round(float(allv.min()), c["decimals"]) >= c["sigma_out_range"][0]
    assert round(float(allv.max()), c["decimals"]) <= c["sigma_out_range"][1]
    # and the band is reached: the scalar map's extremes on [0.01, 1]
    grid = scalar_iterate(np.linspace(lo, hi, 200001), c["K"])
    assert round(float(grid.min()), 2) == c["sigma_out_range"][0]
    assert round(float(grid.max()), 2) == c["sigma_out_range"][1]


def test_worked_deepseek_two_stage_settles():
    c = EX["deepseek_two_stage"]
    table = []
    for n, row in c["stages"]:
        table += [tuple(row)] * n
    U = gen.orthonormal(20, 20, 8)
    V = gen.orthonormal(20, 20, 9)
    s = np.geomspace(1.0, 0.01, 20)
    s = s / np.linalg.norm(s) * 0.999  # pre-scaled values in [0.01, 1)
    s = np.maximum(s, 0.0101)
    out = sv(orc.newton_schulz((U * s) @ V.T, len(table), coeffs=table))
    assert np.all(np.abs(out - c["settles_at"]) < 1e-3)


def test_worked_768_example_oracle_matches_polynomial():
    # The bf16 768x768 example: the fp64 oracle reproduces the scalar
    # polynomial exactly; the GPU bf16 run is held to the printed 0.005.
    c = EX["bf16_768_spectrum"]
    s = np.array(c["sigma_in_head"] + [c["sigma_in_bulk"]] * c["bulk_count"])
    n = c["shape"][0]
    U = gen.orthonormal(n, n, 77)
    V = gen.orthonormal(n, n, 78)
    out = orc.newton_schulz((U * s) @ V.T, c["K"])
    expect = (U * scalar_iterate(s / (np.linalg.norm(s) + 1e-7), c["K"])) @ V.T
    assert np.abs(out - expect).max() < 1e-10


def test_gram_on_wide_side_entry_ratio():
    c = EX["gram_entries_ratio"]
    H, W = c["shape"]
    assert (max(H, W) ** 2) // (min(H, W) ** 2) == c["ratio"]


# ---------------------------------------------------------------------------
# special cases and invariances
# ---------------------------------------------------------------------------

def test_ns_K0_is_prescale():
    X = gen.gaussian((6, 9), 1.0, 3).astype(np.float64)
    got = orc.newton_schulz(X, 0)
    assert np.allclose(got, X / (math.sqrt(float(np.sum(X * X))) + 1e-7), atol=0, rtol=1e-15)


@pytest.mark.parametrize("x", [2.5, -0.3, 1e-3, 0.0])
def test_ns_one_by_one(x):
    got = orc.newton_schulz(np.array([[x]]), 5)[0, 0]
    expect = math.copysign(float(scalar_iterate(abs(x) / (abs(x) + 1e-7), 5)), x) if x != 0 else 0.0
    assert abs(got - expect) < 1e-14


def test_ns_orthogonal_input():
    r = 16
    Q = gen.orthonormal(r, r, 21)
    got = orc.newton_schulz(Q, 5)
    # every pre-scaled singular value is 1 / (sqrt(r) + eps)
    assert np.abs(got - float(scalar_iterate(1.0 / (math.sqrt(r) + 1e-7), 5)) * Q).max() < 1e-13


def test_ns_textbook_cubic_converges_to_polar_factor():
    # (1.5, -0.5, 0) is the classical Newton-Schulz polar iteration: for a full
    # rank input it converges to U V^T (computed here by SVD).
    X = gen.with_singular_values(9, 13, np.linspace(1.0, 0.2, 9), 31)
    got = orc.newton_schulz(X, 80, coeffs=[(1.5, -0.5, 0.0)] * 80)
    U, _, Vt = np.linalg.svd(X, full_matrices=False)
    assert np.abs(got - U @ Vt).max() < 1e-12


@pytest.mark.parametrize("shape", [(8, 8), (6, 11), (11, 6)])
def test_ns_svd_band(shape):
    # Pre-scaled singular values in [0.01, 1] -> outputs in [0.6818, 1.1344],
    # hence ||NS(X) - U V^T||_2 <= 0.3182.
    H, W = shape
    k = min(H, W)
    s = np.concatenate([[1.0], np.linspace(0.3, 0.011, k - 1)])
    X = gen.with_singular_values(H, W, s, 55)
    O = orc.newton_schulz(X, 5)
    assert np.linalg.norm(O - orc.msgn_svd(X), 2) <= 0.3182 + 1e-9


def test_ns_scale_and_transpose_invariance():
    X = gen.gaussian((12, 20), 1.0, 2).astype(np.float64)
    a = orc.newton_schulz(X, 5)
    assert np.abs(orc.newton_schulz(1000.0 * X, 5) - a).max() < 1e-6
    assert np.abs(orc.newton_schulz(X.T, 5) - a.T).max() < 1e-13


def test_momentum_geometric_series():
    G = gen.gaussian((4, 5), 1.0, 9).astype(np.float64)
    beta = 0.95
    M = np.zeros_like(G)
    for n in range(1, 8):
        M = orc.momentum_update(M, G, beta)
        assert np.allclose(M, G * (1 - beta ** n) / (1 - beta), rtol=1e-14, atol=0)


def test_momentum_ema_and_sum_give_same_direction():
    rng_g = [gen.gaussian((10, 16), 1.0, 100 + t).astype(np.float64) for t in range(5)]
    Ms = np.zeros((10, 16))
    Me = np.zeros((10, 16))
    for G in rng_g:
        Ms = orc.momentum_update(Ms, G, 0.9)
        Me = orc.momentum_update_ema(Me, G, 0.9)
    assert np.abs(orc.newton_schulz(Ms, 5) - orc.newton_schulz(Me, 5)).max() < 1e-6


@pytest.mark.parametrize("ema", [False, True])
def test_nesterov_with_zero_beta_is_the_gradient(ema):
    # mu = 0: the blend (1 - mu) G + mu M (or G + mu M) is the fresh gradient
    G = gen.gaussian((6, 9), 1.0, 21).astype(np.float64)
    M0 = gen.gaussian((6, 9), 1.0, 22).astype(np.float64)
    W = gen.gaussian((6, 9), 0.1, 23).astype(np.float64)
    _, _, Os, _ = orc.muonh_step([W], [G], [M0], 0.1, 0.0, 5, [1.0], hook="none", ema=ema, nesterov=True)
    assert np.abs(Os[0] - orc.newton_schulz(G, 5)).max() < 1e-14


@pytest.mark.parametrize("ema,buf,direction", [
    # worked by hand from the Muon explainer's code section with mu = 0.5,
    # G = (1, 0), M0 = (0, 1): the buffer lerps toward G by 1 - mu, the update
    # lerps G toward the buffer by mu
    (True, (0.5, 0.5), (3.0, 1.0)),    # (1-mu)G + mu M1 = (0.75, 0.25)
    # plain-sum buffer: M1 = mu M0 + G = (1, 0.5); look-ahead G + mu M1 = (1.5, 0.25)
    (False, (1.0, 0.5), (6.0, 1.0)),
], ids=["ema", "sum"])
def test_nesterov_worked_example(ema, buf, direction):
    G = np.array([[1.0, 0.0]])
    M0 = np.array([[0.0, 1.0]])
    W = np.array([[0.3, -0.2]])
    _, Ms, Os, _ = orc.muonh_step([W], [G], [M0], 0.1, 0.5, 5, [1.0], hook="none", ema=ema, nesterov=True)
    assert np.array_equal(Ms[0], np.array([buf]))
    d = np.array([direction]) / np.linalg.norm(direction)
    # a row vector keeps its direction through NS (one singular value)
    assert np.abs(Os[0] / np.linalg.norm(Os[0]) - d).max() < 1e-15


def test_nesterov_constant_gradient_keeps_direction():
    # with a constant gradient from M0 = 0 both buffer and blend are positive
    # multiples of G, so the orthogonalized update is NS(G) up to the eps
    G = gen.gaussian((12, 20), 1.0, 31).astype(np.float64)
    M = np.zeros_like(G)
    for _ in range(4):
        W = np.zeros_like(G) + 0.01
        _, Ms, Os, _ = orc.muonh_step([W], [G], [M], 0.1, 0.9, 5, [1.0], hook="none", nesterov=True)
        M = Ms[0]
        assert np.abs(Os[0] - orc.newton_schulz(G, 5)).max() < 1e-6


@pytest.mark.parametrize("H,W,wd", [(16, 16, 0.0), (16, 16, 0.1), (32, 16, 0.05)])
def test_plain_update_closed_form(H, W, wd):
    # G with orthonormal columns (or rows): NS gives p^K(1/(sqrt(r)+eps)) G,
    # and Muon's update is W (1 - eta wd) - eta max(1, H/W)^0.5 O
    Q, _ = np.linalg.qr(gen.gaussian((H, W), 1.0, 41).astype(np.float64))
    r = min(H, W)
    x = scalar_iterate(1.0 / (math.sqrt(r) + 1e-7), 5)
    W0 = gen.gaussian((H, W), 0.02, 42).astype(np.float64)
    eta = 0.02
    Wn, _, Os, _ = orc.muonh_step([W0], [Q], [np.zeros((H, W))], eta, 0.9, 5, [1.0], hook="none",
                                  weight_decay=wd)
    assert np.abs(Os[0] - x * Q).max() < 1e-13
    expect = W0 * (1 - eta * wd) - eta * math.sqrt(max(1.0, H / W)) * x * Q
    assert np.abs(Wn[0] - expect).max() < 1e-14


def test_round_to_bf16_matches_torch():
    torch = pytest.importorskip("torch")
    x = gen.gaussian((1000,), 3.0, 4)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(orc.round_to_bf16(x), ref)


# ---------------------------------------------------------------------------
# Hierarchical Muon
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(20, 36), (36, 20), (32, 32)])
def test_himuon_tile_covering_matrix_equals_full(shape):
    X = gen.gaussian(shape, 1.0, 12).astype(np.float64)
    full = orc.newton_schulz(X, 5)
    tiled = orc.tiled_newton_schulz(X, 40, 5)
    assert np.abs(full - tiled).max() < 1e-12


def test_himuon_unit_tiles_are_elementwise():
    X = gen.gaussian((5, 7), 1.0, 13).astype(np.float64)
    X[2, 3] = 0.0
    got = orc.tiled_newton_schulz(X, 1, 5)
    a = np.abs(X)
    expect = np.sign(X) * scalar_iterate(a / (a + 1e-7), 5)
    assert np.abs(got - expect).max() < 1e-14


def test_himuon_locality_and_per_tile_closed_form():
    T = 8
    H, W = 20, 27  # ragged in both directions
    X = np.zeros((H, W))
    expect = np.zeros((H, W))
    seed = 0
    for r0 in range(0, H, T):
        for c0 in range(0, W, T):
            h, w = min(T, H - r0), min(T, W - c0)
            k = min(h, w)
            s = np.linspace(2.0, 0.1, k)
            U = gen.orthonormal(h, k, 500 + seed)
            V = gen.orthonormal(w, k, 900 + seed)
            seed += 1
            X[r0:r0 + h, c0:c0 + w] = (U * s) @ V.T
            expect[r0:r0 + h, c0:c0 + w] = (U * scalar_iterate(s / (np.linalg.norm(s) + 1e-7), 5)) @ V.T
    got = orc.tiled_newton_schulz(X, T, 5)
    assert np.abs(got - expect).max() < 1e-12
    # perturbing one tile changes that tile only, bit for bit elsewhere
    Y = X.copy()
    Y[9:12, 17:20] += 0.5
    got2 = orc.tiled_newton_schulz(Y, T, 5)
    mask = np.zeros((H, W), bool)
    mask[8:16, 16:24] = True
    assert np.array_equal(got2[~mask], got[~mask])
    assert not np.allclose(got2[mask], got[mask])


def test_himuon_zero_tile_is_zero():
    X = gen.gaussian((16, 16), 1.0, 14).astype(np.float64)
    X[:8, :8] = 0
    assert np.array_equal(orc.tiled_newton_schulz(X, 8, 5)[:8, :8], np.zeros((8, 8)))


# ---------------------------------------------------------------------------
# Hyperball
# ---------------------------------------------------------------------------

def test_hyperball_orthogonal_update_closed_form():
    rho, eta = 3.0, 0.4
    W = np.zeros((6, 8))
    W[:3] = gen.gaussian((3, 8), 1.0, 20)
    W *= rho / np.linalg.norm(W)
    U = np.zeros((6, 8))
    U[3:] = gen.gaussian((3, 8), 1.0, 21) * 7.0  # not unit: Hyperball normalizes it
    U_hat = U / np.linalg.norm(U)
    got, flag = orc.hyperball(W, U, eta, rho)
    assert flag == orc.FLAG_PROJECTED
    assert np.abs(got - rho * (W - eta * U_hat) / math.hypot(rho, eta)).max() < 1e-14


def test_hyperball_angular_step():
    # In the plane of W and U: the new weight turns by atan2(eta sin phi, rho - eta cos phi).
    rho, eta = 2.0, 0.3
    e1 = np.zeros((4, 4)); e1[0, 0] = 1.0
    e2 = np.zeros((4, 4)); e2[1, 2] = 1.0
    for phi in (0.3, 1.2, 2.5):
        U = 5.0 * (math.cos(phi) * e1 + math.sin(phi) * e2)
        got, _ = orc.hyperball(rho * e1, U, eta, rho)
        ang = math.atan2(-got[1, 2], got[0, 0])
        assert abs(ang - math.atan2(eta * math.sin(phi), rho - eta * math.cos(phi))) < 1e-14
        assert abs(np.linalg.norm(got) - rho) < 1e-14


def test_hyperball_radius_invariant_over_steps():
    W0 = gen.gaussian((16, 24), 0.02, 0).astype(np.float64)
    rho = float(np.linalg.norm(W0))
    W = W0
    for t in range(10):
        U = gen.gaussian((16, 24), 1.0, 50 + t)
        W, _ = orc.hyperball(W, U, 0.02, rho)
        assert abs(np.linalg.norm(W) / rho - 1) < 1e-14


def test_hyperball_eta_zero_is_identity_on_sphere():
    W = np.full((4, 4), 0.25)  # ||W|| = 1 exactly
    got, _ = orc.hyperball(W, gen.gaussian((4, 4), 1.0, 1), 0.0, 1.0)
    assert np.array_equal(got, W)


@pytest.mark.parametrize("H,W", [(64, 64), (64, 128)])
def test_hyperball_exact_cancel_restores_radius(H, W):
    W0, G, M0, rho, eta = gen.exact_cancel_case(H, W)
    M = orc.momentum_update(M0, G, 0.95)
    O = orc.newton_schulz(M, 5)
    got, flag = orc.hyperball(W0, O, eta, rho)
    assert flag == orc.FLAG_RESTORED
    # restored along the pre-update weight (W0 is stored in fp32, so its norm
    # is rho up to fp32 rounding)
    W0d = W0.astype(np.float64)
    assert np.abs(got - rho * W0d / np.linalg.norm(W0d)).max() < 1e-15
    assert np.abs(got - W0d).max() < 1e-7 * np.abs(W0d).max()
    assert abs(np.linalg.norm(got) - rho) < 1e-12


def test_hyperball_zero_weight_fixed_radius():
    U = gen.gaussian((5, 6), 1.0, 2).astype(np.float64)
    got, flag = orc.hyperball(np.zeros((5, 6)), U, 0.1, 2.0)
    assert flag == orc.FLAG_PROJECTED
    assert np.abs(got + 2.0 * U / np.linalg.norm(U)).max() < 1e-14


def test_hyperball_zero_everything_unrestorable():
    got, flag = orc.hyperball(np.zeros((3, 3)), np.zeros((3, 3)), 0.1, 1.0)
    assert flag == orc.FLAG_UNRESTORABLE and not got.any()


def test_hyperball_zero_update_projects_only():
    W = gen.gaussian((3, 7), 1.0, 3).astype(np.float64)
    got, flag = orc.hyperball(W, np.zeros((3, 7)), 0.5, 4.0)
    assert flag == orc.FLAG_PROJECTED
    assert np.allclose(got, 4.0 * W / np.linalg.norm(W), rtol=1e-15, atol=0)


def test_hyperball_radius_step_turns_by_atan_eta():
    # Radius-sized step: for an update orthogonal to W the weight turns by
    # atan(eta) whatever rho is (the unit step turns by atan(eta / rho)).
    eta = 0.3
    e1 = np.zeros((3, 5)); e1[0, 1] = 1.0
    e2 = np.zeros((3, 5)); e2[2, 4] = 1.0
    for rho in (0.5, 2.0, 7.0):
        got, flag = orc.hyperball(rho * e1, 9.0 * e2, eta, rho, step="radius")
        assert flag == orc.FLAG_PROJECTED
        assert abs(math.atan2(-got[2, 4], got[0, 1]) - math.atan(eta)) < 1e-14
        unit, _ = orc.hyperball(rho * e1, 9.0 * e2, eta, rho)
        assert abs(math.atan2(-unit[2, 4], unit[0, 1]) - math.atan(eta / rho)) < 1e-14
        assert abs(np.linalg.norm(got) - rho) < 1e-14


def test_hyperball_radius_step_is_unit_step_at_unit_radius():
    W = gen.gaussian((6, 9), 1.0, 30).astype(np.float64)
    W /= np.linalg.norm(W)
    U = gen.gaussian((6, 9), 1.0, 31)
    a, _ = orc.hyperball(W, U, 0.05, 1.0)
    b, _ = orc.hyperball(W, U, 0.05, 1.0, step="radius")
    assert np.array_equal(a, b)


def test_hyperball_radius_step_exact_cancel_restores():
    # W = eta * rho * U_hat cancels exactly under the radius step.
    rho, eta = 2.0, 0.5
    U = np.zeros((4, 4)); U[1, 3] = 3.0
    W = np.zeros((4, 4)); W[1, 3] = eta * rho
    got, flag = orc.hyperball(W, U, eta, rho, step="radius")
    assert flag == orc.FLAG_RESTORED
    assert got[1, 3] == rho and np.count_nonzero(got) == 1


def test_relative_update_worked_example():
    # ||W|| = 5, O along the second coordinate: W - 0.1 * 5 * (0, 1)
    got = orc.relative_update(np.array([[3.0, 4.0]]), np.array([[0.0, 2.0]]), 0.1)
    assert np.array_equal(got, np.array([[3.0, 3.5]]))


def test_relative_update_step_length_and_direction():
    W = gen.gaussian((12, 20), 0.02, 32).astype(np.float64)
    O = gen.gaussian((12, 20), 1.0, 33).astype(np.float64)
    eta = 0.07
    got = orc.relative_update(W, O, eta)
    d = got - W
    assert abs(np.linalg.norm(d) - eta * np.linalg.norm(W)) < 1e-15
    cos = -np.sum(d * O) / (np.linalg.norm(d) * np.linalg.norm(O))
    assert abs(cos - 1) < 1e-14
    # invariant to the scale of O (so also to Muon's shape scale)
    assert np.allclose(orc.relative_update(W, 3.7 * O, eta), got, rtol=0, atol=1e-17)


def test_relative_update_zero_update_and_zero_weight():
    W = gen.gaussian((3, 4), 1.0, 34).astype(np.float64)
    assert np.array_equal(orc.relative_update(W, np.zeros((3, 4)), 0.1), W)
    # a zero weight takes no step (its norm sets the step length)
    assert not orc.relative_update(np.zeros((3, 4)), W, 0.1).any()


def test_step_relative_hook_composes_the_pieces():
    W = gen.gaussian((8, 12), 0.02, 35).astype(np.float64)
    G = gen.gaussian((8, 12), 0.02, 36).astype(np.float64)
    M = np.zeros((8, 12))
    nw, nm, Os, _ = orc.muonh_step([W], [G], [M], 0.02, 0.95, 5, [1.0], hook="relative")
    m = orc.momentum_update(M, G, 0.95)
    assert np.array_equal(nw[0], orc.relative_update(W, orc.newton_schulz(m, 5), 0.02))


def test_frob_project_plain():
    W = gen.gaussian((3, 7), 1.0, 4).astype(np.float64)
    got, _ = orc.frob_project(W, None, 0.1, 2.5)
    assert np.allclose(got, 2.5 * W / np.linalg.norm(W), rtol=1e-15, atol=0)


# ---------------------------------------------------------------------------
# RadialBrake
# ---------------------------------------------------------------------------

def _rb_case(c, H=3, W=4):
    # w_prev of norm norm_prev along a 3-4-5 direction; an update that scales it
    # to norm_after_update.
    d = np.zeros((H, W)); d[0, 0] = 3.0; d[1, 1] = 4.0  # norm 5
    Wp = d * (c["norm_prev"] / 5.0)
    target = d * (c["norm_after_update"] / 5.0)
    eta = 0.5
    O = (Wp - target) / (eta * orc.shape_scale(H, W))
    return Wp, O, eta


@pytest.mark.parametrize("c", HB["radial_brake"], ids=lambda c: c["id"])
def test_radial_brake_norm_rule(c):
    Wp, O, eta = _rb_case(c)
    got = orc.radial_brake(Wp, O, eta, c["outward"], c["inward"])
    assert abs(np.linalg.norm(got) - c["norm_expected"]) < 1e-13
    # the direction is the optimizer's updated weight
    tgt = Wp * (c["norm_after_update"] / c["norm_prev"])
    assert np.abs(got / np.linalg.norm(got) - tgt / np.linalg.norm(tgt)).max() < 1e-14


def test_radial_brake_shape_scale_on_tall_matrix():
    H, W = 8, 2
    Wp = gen.gaussian((H, W), 1.0, 1).astype(np.float64)
    O = gen.gaussian((H, W), 1.0, 2).astype(np.float64)
    got = orc.radial_brake(Wp, O, 0.1, 1.0, 1.0)  # s = 1: no braking
    assert np.abs(got - (Wp - 0.1 * 2.0 * O)).max() < 1e-14


def test_radial_brake_zero_post_norm_leaves_update():
    Wp = np.ones((2, 2))
    got = orc.radial_brake(Wp, Wp / 0.5, 0.5, 0.5, 0.5)
    assert not got.any()


# ---------------------------------------------------------------------------
# full step
# ---------------------------------------------------------------------------

def test_step_composes_parts():
    W0, Gs, M0 = gen.single_matrix_case(16, 24, steps=3)
    W = W0.astype(np.float64)
    rho = float(np.linalg.norm(W))
    M = M0.astype(np.float64)
    Ws, Ms = [W], [M]
    for G in Gs:
        Ws, Ms, Os, flags = orc.muonh_step(Ws, [G], Ms, 0.02, 0.95, 5, [rho])
        assert abs(np.linalg.norm(Ws[0]) / rho - 1) < 1e-14
    M_ref = np.zeros((16, 24))
    for G in Gs:
        M_ref = 0.95 * M_ref + G
    assert np.allclose(Ms[0], M_ref, rtol=1e-15, atol=1e-18)


# ---------------------------------------------------------------------------
# planted mistakes: each variant must fail at least one pin above
# ---------------------------------------------------------------------------

def _ns_variant(kind):
    def fn(G, K):
        X = np.array(G, dtype=np.float64)
        tall = X.shape[0] > X.shape[1]
        if tall and kind != "no_transpose":
            X = X.T
        X = X / (np.linalg.norm(X) + 1e-7)
        a, b, c = ABC
        for _ in range(K):
            if kind == "gram_wrong_side":
                A = X.T @ X
                B = b * A + c * (A @ A)
                X = a * X + X @ B
                continue
            A = X @ X.T
            if kind == "dropped_c":
                B = b * A
            elif kind == "sign_b":
                B = -b * A + c * (A @ A)
            else:
                B = b * A + c * (A @ A)
            X = a * X + B @ X
        if tall and kind not in ("no_transpose", "no_transpose_back"):
            X = X.T
        return X
    return fn


@pytest.mark.parametrize("kind", ["dropped_c", "sign_b", "no_transpose_back"])
@pytest.mark.filterwarnings("ignore::RuntimeWarning")
def test_planted_mistakes_fail_closed_form(kind):
    errs = [closed_form_error(_ns_variant(kind), H, W, 5, 1) for H, W in [(7, 5), (5, 7)]]
    assert max(errs) > 1e-3


def test_planted_wrong_side_gram_is_only_a_cost_change():
    # Using the tall-side Gram is mathematically the same map (p is odd), so
    # the closed form holds: the pages' wide-side rule is about cost only.
    assert closed_form_error(_ns_variant("gram_wrong_side"), 7, 5, 5, 1) < 1e-12


def test_planted_unnormalized_update_fails_hyperball_pin():
    rho, eta = 3.0, 0.4
    W = np.zeros((2, 2)); W[0, 0] = rho
    U = np.zeros((2, 2)); U[1, 1] = 7.0
    wrong = rho * (W - eta * U) / np.linalg.norm(W - eta * U)
    good, _ = orc.hyperball(W, U, eta, rho)
    expect = rho * (W - eta * U / 7.0) / math.hypot(rho, eta)
    assert np.abs(good - expect).max() < 1e-14
    assert np.abs(wrong - expect).max() > 1e-2


# ---------------------------------------------------------------------------
# AdamH
# ---------------------------------------------------------------------------

def test_adam_first_step_is_sign_like():
    # From zero moments the bias corrections give m_hat = g, v_hat = g^2, so
    # U = g / (|g| + eps) exactly.
    G = gen.gaussian((5, 7), 1e-3, 40).astype(np.float64)
    m, v, U = orc.adam_direction(np.zeros((5, 7)), np.zeros((5, 7)), G, 0.9, 0.95, 1e-8, 1)
    assert np.allclose(U, G / (np.abs(G) + 1e-8), rtol=1e-14, atol=0)
    assert np.allclose(m, 0.1 * G, rtol=1e-15, atol=0) and np.allclose(v, 0.05 * G * G, rtol=1e-15, atol=0)


def test_adam_constant_gradient_bias_correction_is_exact():
    # m_t = (1 - b1^t) g and v_t = (1 - b2^t) g^2: the corrected ratio stays g / (|g| + eps)
    G = np.array([[2e-3, -5e-4], [1e-3, 3e-3]])
    M = np.zeros_like(G); V = np.zeros_like(G)
    for t in range(1, 9):
        M, V, U = orc.adam_direction(M, V, G, 0.9, 0.95, 1e-8, t)
        assert np.allclose(M, (1 - 0.9 ** t) * G, rtol=1e-13, atol=0)
        assert np.allclose(V, (1 - 0.95 ** t) * G * G, rtol=1e-13, atol=0)
        assert np.allclose(U, G / (np.abs(G) + 1e-8), rtol=1e-12, atol=0)


def test_adam_worked_numbers():
    # one coordinate by hand: m = 0.9*0.2 + 0.1*0.5 = 0.23, v = 0.95*0.04 + 0.05*0.25 = 0.0505,
    # t = 2: U = (0.23/0.19) / (sqrt(0.0505/0.0975) + 1e-8)
    m, v, U = orc.adam_direction(np.array([[0.2]]), np.array([[0.04]]), np.array([[0.5]]), 0.9, 0.95, 1e-8, 2)
    assert abs(m[0, 0] - 0.23) < 1e-15 and abs(v[0, 0] - 0.0505) < 1e-15
    assert abs(U[0, 0] - (0.23 / 0.19) / (math.sqrt(0.0505 / 0.0975) + 1e-8)) < 1e-14


def test_adamh_keeps_radius_and_steps_along_minus_u():
    W = gen.gaussian((16, 24), 0.02, 41).astype(np.float64)
    rho = float(np.linalg.norm(W))
    G = gen.gaussian((16, 24), 1e-3, 42)
    nw, nm, nv, Us, fl = orc.adamh_step([W], [G], [np.zeros((16, 24))], [np.zeros((16, 24))], 0.02, 0.9, 0.95,
                                        1e-8, 1, [rho])
    assert fl[0] == orc.FLAG_PROJECTED
    assert abs(np.linalg.norm(nw[0]) - rho) < 1e-13
    # same as the Hyperball of the Adam direction
    ref, _ = orc.hyperball(W, Us[0], 0.02, rho)
    assert np.array_equal(nw[0], ref)


def test_adamw_closed_form_first_step():
    W = gen.gaussian((6, 9), 0.02, 43).astype(np.float64)
    G = gen.gaussian((6, 9), 1e-3, 44).astype(np.float64)
    Z = np.zeros((6, 9))
    nw, _, _, _, _ = orc.adamh_step([W], [G], [Z], [Z], 0.01, 0.9, 0.95, 1e-8, 1, hook="none", weight_decay=0.1,
                                    state_f32=False)
    assert np.allclose(nw[0], W * (1 - 0.001) - 0.01 * G / (np.abs(G) + 1e-8), rtol=1e-14, atol=1e-18)


def test_adamh_zero_gradient_projects_only():
    W = gen.gaussian((4, 4), 1.0, 45).astype(np.float64)
    Z = np.zeros((4, 4))
    nw, _, _, Us, fl = orc.adamh_step([W], [Z], [Z], [Z], 0.1, 0.9, 0.95, 1e-8, 1, [3.0])
    assert not Us[0].any() and fl[0] == orc.FLAG_PROJECTED
    assert np.allclose(nw[0], 3.0 * W / np.linalg.norm(W), rtol=1e-15, atol=0)


def test_adam_hooks_match_the_muon_hooks_without_shape_scale():
    # wide matrix: Muon's shape scale is 1, so the brake and the relative step
    # of the Adam direction equal the stand-alone hooks applied to U
    W = gen.gaussian((6, 10), 0.02, 46).astype(np.float64)
    G = gen.gaussian((6, 10), 1e-3, 47).astype(np.float64)
    Z = np.zeros((6, 10))
    for hook, ref in (("radial_brake", lambda U: orc.radial_brake(W, U, 0.02)),
                      ("relative", lambda U: orc.relative_update(W, U, 0.02))):
        nw, _, _, Us, _ = orc.adamh_step([W], [G], [Z], [Z], 0.02, 0.9, 0.95, 1e-8, 3, hook=hook)
        assert np.array_equal(nw[0], ref(Us[0]))


def test_step_per_matrix_tile_sizes_route_each_matrix():
    shapes = [(40, 70), (64, 32), (50, 50)]
    sizes = [0, 16, 32]
    Ws = [gen.gaussian(sh, 0.02, 60 + i).astype(np.float64) for i, sh in enumerate(shapes)]
    Gs = [gen.gaussian(sh, 0.02, 70 + i).astype(np.float64) for i, sh in enumerate(shapes)]
    Ms = [np.zeros(sh) for sh in shapes]
    rhos = [float(np.linalg.norm(w)) for w in Ws]
    nw, _, Os, _ = orc.muonh_step(Ws, Gs, Ms, 0.02, 0.95, 5, rhos, tile_sizes=sizes)
    for i in range(3):
        one, _, O1, _ = orc.muonh_step([Ws[i]], [Gs[i]], [Ms[i]], 0.02, 0.95, 5, [rhos[i]], tile_T=sizes[i])
        assert np.array_equal(nw[i], one[0]) and np.array_equal(Os[i], O1[0])
