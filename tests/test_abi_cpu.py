"""Host-side checks of the C ABI (no GPU needed, no compute call):
the library loads, exports every function the header declares, rejects bad
arguments before touching the GPU, and the host planner's accounting matches
the closed-form work counts."""
import ctypes
import os
import re

import pytest

import matrix_orthogonalizing_optimizer_momentum_amd as mm
from synth import gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muonh.h")

pytestmark = pytest.mark.skipif(not os.path.exists(mm.LIB_PATH), reason="libmuonh.so not built")


def header_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_ \*]*?\b([a-z_][a-z0-9_]*)\s*\(", txt, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


def test_header_declares_the_entry_points():
    names = header_functions()
    for n in ("muonh_step", "ns_orthogonalize", "frob_project", "muonh_strerror", "muonh_get_flags",
              "muonh_release", "muonh_plan_query", "adamh_step"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(mm.LIB_PATH)
    for n in header_functions():
        assert hasattr(lib, n), n
    assert set(header_functions()) == set(mm.EXPORTED)


def test_strerror_and_version():
    assert mm.strerror(mm.MUONH_OK) == "success"
    assert "invalid" in mm.strerror(mm.MUONH_EINVAL)
    assert mm.strerror(-99) == "unknown error"
    assert "gfx950" in mm.version()


def _opts():
    o = mm.Opts()
    mm.load().muonh_default_opts(ctypes.byref(o))
    return o


def _step(n=1, shapes=(4, 4), eta=0.02, beta=0.95, K=5, rho=1.0, tile=0, ptr=0x1000, opts=None, null_rho=False):
    lib = mm.load()
    P = ctypes.c_void_p * max(n, 1)
    ps = P(*[ptr + 0x100 * i for i in range(max(n, 1))])
    gs = P(*[ptr + 0x10000 + 0x100 * i for i in range(max(n, 1))])
    ms = P(*[ptr + 0x20000 + 0x100 * i for i in range(max(n, 1))])
    sh = (ctypes.c_int64 * (2 * max(n, 1)))(*(list(shapes) * max(n, 1)))
    rh = None if null_rho else (ctypes.c_float * max(n, 1))(*([rho] * max(n, 1)))
    o = opts or _opts()
    return lib.muonh_step(ps, gs, ms, sh, n, eta, beta, K, rh, tile, ctypes.byref(o))


# Each of these is rejected by host validation, before any HIP call.
@pytest.mark.parametrize("kw", [
    dict(n=0), dict(K=-1), dict(K=65), dict(beta=1.0), dict(beta=-0.1), dict(eta=-1.0),
    dict(eta=float("nan")), dict(rho=0.0), dict(rho=float("inf")), dict(null_rho=True),
    dict(shapes=(0, 4)), dict(shapes=(4, -2)), dict(tile=-1), dict(tile=8256), dict(tile=200),
])
def test_step_validation_rejects(kw):
    assert _step(**kw) == mm.MUONH_EINVAL


def test_step_rejects_bad_options():
    for field, val in [("state_dtype", 7), ("ns_dtype", 3), ("ns_precision", 9), ("hook", 5),
                       ("outward", 1.5), ("inward", -0.1), ("ns_eps", float("nan")), ("momentum_ema", 2),
                       ("nesterov", -1), ("weight_decay", -0.5), ("weight_decay", float("inf")),
                       ("lanes", -1), ("lanes", 5), ("hook", 4), ("hyperball_step", 2),
                       ("param_dtype", 1), ("param_dtype", 7), ("deterministic", 2), ("deterministic", -1)]:
        o = _opts()
        setattr(o, field, val)
        assert _step(opts=o) == mm.MUONH_EINVAL, field


def test_default_options():
    o = _opts()
    assert (o.state_dtype, o.ns_dtype, o.ns_precision, o.hook) == (mm.MUONH_BF16, mm.MUONH_BF16, mm.MUONH_NS_H16,
                                                                   mm.MUONH_HOOK_HYPERBALL)
    assert (o.momentum_ema, o.nesterov, o.weight_decay, o.workspace_limit, o.lanes) == (0, 0, 0.0, 0, 0)
    assert o.hyperball_step == mm.MUONH_HB_STEP_UNIT
    assert abs(o.ns_eps - 1e-7) < 1e-12 and abs(o.zero_rel_eps - 1e-6) < 1e-11
    assert (o.outward, o.inward) == (0.5, 1.0)
    assert (o.param_dtype, o.deterministic) == (mm.MUONH_F32, 1)


def test_enums_follow_the_boundary_contract():
    # MUONH_NS_FOLD = 0 (bf16 X, folded pre-scale), MUONH_NS_X32 = 1, as the
    # boundary numbers them, and MUONH_NS_H16 = 2 after them, as the header
    # declares them
    import re
    hdr = open(HEADER).read()
    m = re.search(r"enum\s*\{\s*MUONH_NS_FOLD\s*=\s*(\d+),\s*MUONH_NS_X32\s*=\s*(\d+),\s*MUONH_NS_H16\s*=\s*(\d+)\s*\}",
                  hdr)
    got = tuple(int(m.group(i)) for i in (1, 2, 3)) if m else None
    assert got == (mm.MUONH_NS_FOLD, mm.MUONH_NS_X32, mm.MUONH_NS_H16) == (0, 1, 2)


def test_lanes_share_one_chunk_workspace():
    # Concurrent lanes carve disjoint regions out of what one chunk would use.
    shapes = [(768, 2304), (768, 768), (768, 3072), (3072, 768)] * 3
    q = mm.plan_query(shapes, K=5)
    assert q["chunks"] == 1 and q["lanes"] == 2
    assert q["ws_bytes"] == sum(mm.plan_query([sh], K=5)["ws_bytes"] for sh in shapes)
    assert mm.plan_query(shapes, K=5, lanes=4)["lanes"] == 4
    assert mm.plan_query(shapes[:3], K=5, lanes=4)["lanes"] == 3  # never more lanes than matrices
    assert mm.plan_query(shapes, K=5, lanes=1)["lanes"] == 1
    assert mm.plan_query(shapes[:1], K=5)["lanes"] == 1


def test_automatic_lanes_follow_iteration_work():
    # Two lanes, but one for NS on the GEMM engine (full matrices, or tiles
    # above the resident sizes) whose iteration exceeds 2e12 flops, and one
    # when every matrix runs as resident tiles.
    small = [(1024, 1024)] * 4   # 4 * 6 * 1024^3 flops per iteration
    big = [(8192, 8192)] * 2     # 2 * 6 * 8192^3 > 2e12
    assert mm.plan_query(small, K=5)["lanes"] == 2
    assert mm.plan_query(big, K=5)["lanes"] == 1
    assert mm.plan_query(big, K=5, tile_T=128)["lanes"] == 1   # resident tiles
    assert mm.plan_query(small, K=5, tile_T=64)["lanes"] == 1
    huge = [(16384, 16384)] * 8  # 8 * 4096 tiles of 256^2: 3.3e12 flops per iteration
    # bf16 tiles of 256 run fused (resident): one lane; with the fp32 master
    # copy (X32) they go through the GEMM engine: one lane for this iteration
    # size, two for a small one
    assert mm.plan_query(huge, K=5, tile_T=256, workspace_limit=1 << 40)["lanes"] == 1
    assert mm.plan_query(huge, K=5, tile_T=256, workspace_limit=1 << 40, ns_precision="x32")["lanes"] == 1
    assert mm.plan_query(big, K=5, tile_T=256, workspace_limit=1 << 40, ns_precision="x32")["lanes"] == 2  # 2.1e11
    assert mm.plan_query(big, K=5, lanes=2)["lanes"] == 2
    # a budget that forces sequential chunks leaves no room for lanes
    one = mm.plan_query(small[:1], K=5)["ws_bytes"]
    q = mm.plan_query(small, K=5, workspace_limit=2 * one)
    assert q["chunks"] == 2 and q["lanes"] == 1


def test_plain_update_needs_no_radius_and_no_hook_pass():
    # Muon's own update: rho may be NULL, and the plan has no Hyperball pass 1
    o = _opts()
    o.hook = mm.MUONH_HOOK_NONE
    q_hb = mm.plan_query([(64, 64)], K=5)  # default hook: Hyperball
    assert q_hb["stream_bytes"] == 64 * 64 * 22  # momentum 6, hook pass 1 6, update pass 10
    # resident tiles sum the hook's norms where O is stored: a W read (4) instead of pass 1
    assert mm.plan_query([(64, 64)], K=5, tile_T=64)["stream_bytes"] == 64 * 64 * 20
    lib = mm.load()
    out = (ctypes.c_int64 * 7)()
    sh = (ctypes.c_int64 * 2)(64, 64)
    assert lib.muonh_plan_query(sh, 1, 5, 0, ctypes.byref(o), 0, out) == mm.MUONH_OK
    assert out[5] == 64 * 64 * 16  # 6 (momentum) + 10 (update pass)


def test_relative_update_needs_no_radius_and_reads_only_w_in_pass_one():
    o = _opts()
    o.hook = mm.MUONH_HOOK_RELATIVE
    lib = mm.load()
    out = (ctypes.c_int64 * 7)()
    sh = (ctypes.c_int64 * 2)(64, 64)
    assert lib.muonh_plan_query(sh, 1, 5, 0, ctypes.byref(o), 0, out) == mm.MUONH_OK
    assert out[5] == 64 * 64 * 20  # 6 (momentum) + 4 (W read for ||W||^2) + 10 (update pass)


def test_step_rejects_null_pointers_and_aliasing():
    lib = mm.load()
    o = _opts()
    P = ctypes.c_void_p * 1
    sh = (ctypes.c_int64 * 2)(4, 4)
    rh = (ctypes.c_float * 1)(1.0)
    assert lib.muonh_step(P(None), P(0x1000), P(0x2000), sh, 1, 0.1, 0.9, 5, rh, 0, ctypes.byref(o)) == mm.MUONH_EINVAL
    assert lib.muonh_step(P(0x1000), P(0x2000), P(0x2000), sh, 1, 0.1, 0.9, 5, rh, 0, ctypes.byref(o)) == mm.MUONH_EINVAL
    assert lib.muonh_step(None, P(0x2000), P(0x3000), sh, 1, 0.1, 0.9, 5, rh, 0, ctypes.byref(o)) == mm.MUONH_EINVAL


def test_coefficient_table_must_be_finite():
    o = _opts()
    arr = (ctypes.c_float * 15)(*([3.4445, -4.775, 2.0315] * 4 + [float("nan"), 0, 0]))
    o.coeffs = ctypes.cast(arr, ctypes.POINTER(ctypes.c_float))
    assert _step(opts=o, K=5) == mm.MUONH_EINVAL


def test_ns_and_projection_validation():
    lib = mm.load()
    o = _opts()
    P = ctypes.c_void_p * 1
    sh = (ctypes.c_int64 * 2)(4, 4)
    assert lib.ns_orthogonalize(P(None), P(0x1000), sh, 1, 5, 0, ctypes.byref(o)) == mm.MUONH_EINVAL
    assert lib.ns_orthogonalize(P(0x1000), P(0x2000), sh, 1, 99, 0, ctypes.byref(o)) == mm.MUONH_EINVAL
    rh = (ctypes.c_float * 1)(-1.0)
    assert lib.frob_project(P(0x1000), None, sh, 1, 0.1, rh, ctypes.byref(o)) == mm.MUONH_EINVAL
    rh = (ctypes.c_float * 1)(1.0)
    assert lib.frob_project(P(0x1000), None, sh, 1, float("inf"), rh, ctypes.byref(o)) == mm.MUONH_EINVAL


def _dense_flops(shapes, K):
    tot = 0
    for H, W in shapes:
        r, s = min(H, W), max(H, W)
        tot += K * (4 * r * r * s + 2 * r ** 3)
    return tot


def test_plan_query_gpt2_accounting():
    shapes = gen.gpt2_small_shapes()
    q = mm.plan_query(shapes, K=5)
    assert q["chunks"] == 1 and q["units"] == 48
    assert q["ns_flops"] == _dense_flops(shapes, 5)
    elems = sum(H * W for H, W in shapes)
    # bf16 state, bf16 operands: momentum 6 B + hook pass 1 (4 + 2) + pass 2 (4 + 2 + 4) = 22 B/elem
    assert q["stream_bytes"] == 22 * elems


def test_plan_query_tiled_units_and_flops():
    shapes = [(300, 700), (768, 2304)]
    q = mm.plan_query(shapes, K=5, tile_T=128)
    assert q["units"] == 3 * 6 + 6 * 18
    tot = 0
    for H, W in shapes:
        for r0 in range(0, H, 128):
            for c0 in range(0, W, 128):
                h, w = min(128, H - r0), min(128, W - c0)
                a, b = min(h, w), max(h, w)
                tot += 5 * (4 * a * a * b + 2 * a ** 3)
    assert q["ns_flops"] == tot


@pytest.mark.parametrize("T", [1, 37, 64, 96, 128])
def test_plan_query_resident_tiles(T):
    # T <= 128: one workgroup per tile for the whole step; the only workspace
    # is the step's orthogonalized-update buffer (bf16, 256-byte aligned).
    shapes = [(300, 700), (768, 2304)]
    q = mm.plan_query(shapes, K=5, tile_T=T)
    tiles = sum(-(-H // T) * -(-W // T) for H, W in shapes)
    assert q["units"] == tiles and q["jobs_per_iter"] == tiles
    assert q["ws_bytes"] == sum(-(-H * W * 2 // 256) * 256 for H, W in shapes)
    assert q["chunks"] == 1


def test_plan_query_fused_256_tiles_need_only_the_output():
    # bf16 tiles of 129..256 run on the fused kernel: no Newton-Schulz
    # workspace, only the step's bf16 O buffer; the fp32 master copy sends
    # them to the GEMM engine, which needs per-tile workspace
    shapes = [(768, 2304), (3072, 768)]
    numel = sum(h * w for h, w in shapes)
    for T in (192, 256):
        assert mm.plan_query(shapes, K=5, tile_T=T, lanes=1)["ws_bytes"] <= 2 * numel + 2 * 256
        assert mm.plan_query(shapes, K=5, tile_T=T, lanes=1, ns_precision="x32")["ws_bytes"] > 4 * numel


def test_plan_query_gemm_engine_tiles_need_workspace():
    # T > 256, or 128 < T <= 256 without the fused kernel's conditions (here
    # the fp32 master copy), runs through the GEMM engine with per-tile workspace.
    shapes = [(768, 2304)]
    assert mm.plan_query(shapes, K=5, tile_T=512)["ws_bytes"] > mm.plan_query(shapes, K=5, tile_T=128)["ws_bytes"]
    assert (mm.plan_query(shapes, K=5, tile_T=256, ns_precision="x32")["ws_bytes"] >
            mm.plan_query(shapes, K=5, tile_T=256)["ws_bytes"])


def test_small_fp32_units_run_on_64_tiles():
    # fp32 operands with r <= 256 take 64 x 64 output tiles: upper tiles of
    # G1 and G2 (4 * 5 / 2 each) plus all 16 of G3 at 256 x 256; bf16 and
    # larger fp32 units keep 128-tiles (3 + 3 + 4 at 256 x 256).
    assert mm.plan_query([(256, 256)], K=5, ns_dtype="f32")["jobs_per_iter"] == 10 + 10 + 16
    assert mm.plan_query([(256, 256)], K=5, ns_dtype="bf16")["jobs_per_iter"] == 3 + 3 + 4
    assert mm.plan_query([(64, 128)], K=5, ns_dtype="f32")["jobs_per_iter"] == 1 + 1 + 2
    assert mm.plan_query([(384, 384)], K=5, ns_dtype="f32")["jobs_per_iter"] == 6 + 6 + 9


def test_plan_query_chunking_under_a_budget():
    shapes = gen.gpt2_small_shapes()
    one = mm.plan_query(shapes[:1], K=5)["ws_bytes"]
    q = mm.plan_query(shapes, K=5, workspace_limit=3 * one)
    assert q["chunks"] > 1 and q["ws_bytes"] <= 3 * one
    with pytest.raises(mm.MuonhError) as e:
        mm.plan_query([(3072, 768)], K=5, workspace_limit=1024)
    assert e.value.code == mm.MUONH_ENOMEM


def _min_max_partition(b, parts):
    """Smallest achievable largest sum when b is cut into `parts` runs (DP)."""
    n = len(b)
    pre = [0]
    for v in b:
        pre.append(pre[-1] + v)
    INF = float("inf")
    best = [[INF] * (n + 1) for _ in range(parts + 1)]
    best[0][0] = 0
    for k in range(1, parts + 1):
        for j in range(1, n + 1):
            for i in range(k - 1, j):
                best[k][j] = min(best[k][j], max(best[k - 1][i], pre[j] - pre[i]))
    return best[parts][n]


def _greedy_count(b, limit):
    count, acc = 1, 0
    for v in b:
        if acc + v > limit and acc > 0:
            count, acc = count + 1, 0
        acc += v
    return count


def test_chunks_are_fewest_and_balanced():
    # The chunk count is the fewest that fit the budget, and the largest chunk
    # is the smallest any cut into that many runs of consecutive matrices allows.
    import random
    rng = random.Random(7)
    shapes = [(rng.choice([128, 384, 768, 1024, 2048]), rng.choice([256, 768, 3072])) for _ in range(14)]
    b = [mm.plan_query([s], K=5)["ws_bytes"] for s in shapes]
    total = mm.plan_query(shapes, K=5, lanes=1)["ws_bytes"]
    assert total == sum(b)
    for limit in (max(b), max(b) + 1, 2 * max(b), total // 3, total // 2, total - 1):
        if limit < max(b):
            continue
        q = mm.plan_query(shapes, K=5, workspace_limit=limit)
        want = _greedy_count(b, limit)
        assert q["chunks"] == want, limit
        if want > 1:
            assert q["ws_bytes"] == _min_max_partition(b, want), limit
    # Eight-layer chunks of the 8B-shaped set under a 16 GiB budget, not
    # three chunks of ten layers and a short last one.
    layer = [(4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096), (4096, 14336), (4096, 14336), (14336, 4096)]
    q16 = mm.plan_query(layer * 32, K=5, workspace_limit=16 << 30)
    assert q16["chunks"] == 4
    assert q16["ws_bytes"] == 8 * mm.plan_query(layer, K=5, lanes=1)["ws_bytes"]


def test_x32_needs_more_workspace_than_fold():
    s = [(768, 3072)]
    assert mm.plan_query(s, ns_precision="x32")["ws_bytes"] > mm.plan_query(s, ns_precision="fold")["ws_bytes"]


def test_fp16_iterates_need_the_workspace_of_bf16_x():
    # fp16 iterates take the place of the bf16 ones: same buffers, same bytes,
    # the same chunks under a budget (the 8B-shaped set at 16 GiB: 4 chunks)
    from synth import gen
    for shapes, limit in (([(768, 3072), (3072, 768), (300, 700)], 0), (gen.dense_8b_shapes(), 16 << 30)):
        h = mm.plan_query(shapes, ns_precision="h16", workspace_limit=limit)
        f = mm.plan_query(shapes, ns_precision="fold", workspace_limit=limit)
        assert h["ws_bytes"] == f["ws_bytes"] and h["chunks"] == f["chunks"]
    assert mm.plan_query(gen.dense_8b_shapes(), workspace_limit=16 << 30)["chunks"] == 4


def test_precision_option_is_validated():
    o = _opts()
    for bad in (3, -1):
        o.ns_precision = bad
        P = ctypes.c_void_p * 1
        rc = mm.load().ns_orthogonalize(P(0x1000), P(0x2000), (ctypes.c_int64 * 2)(8, 8), 1, 5, 0, ctypes.byref(o))
        assert rc == mm.MUONH_EINVAL


def _adam(n=1, eta=0.01, b1=0.9, b2=0.95, eps=1e-8, step=1, null_rho=False, alias=None, opts=None):
    lib = mm.load()
    P = ctypes.c_void_p * max(n, 1)
    ps, gs = P(*([0x1000] * max(n, 1))), P(*([0x2000] * max(n, 1)))
    ms = P(*([0x3000] * max(n, 1)))
    vs = P(*([0x3000 if alias == "mv" else 0x4000] * max(n, 1)))
    if alias == "gm":
        ms = P(*([0x2000] * max(n, 1)))
    sh = (ctypes.c_int64 * (2 * max(n, 1)))(*([8, 8] * max(n, 1)))
    rh = None if null_rho else (ctypes.c_float * max(n, 1))(*([1.0] * max(n, 1)))
    o = opts or _opts()
    return lib.adamh_step(ps, gs, ms, vs, sh, n, eta, b1, b2, eps, step, rh, ctypes.byref(o))


# Each of these is rejected by host validation, before any HIP call.
@pytest.mark.parametrize("kw", [
    dict(n=0), dict(eta=-1.0), dict(b1=1.0), dict(b2=-0.1), dict(eps=0.0), dict(eps=float("nan")),
    dict(step=0), dict(null_rho=True), dict(alias="mv"), dict(alias="gm"),
])
def test_adamh_validation_rejects(kw):
    assert _adam(**kw) == mm.MUONH_EINVAL


def test_adamh_rejects_bad_hook_option():
    o = _opts()
    o.hook = 9
    assert _adam(opts=o) == mm.MUONH_EINVAL


def test_per_matrix_tile_sizes_plan():
    shapes = [(768, 2304), (768, 768), (768, 3072), (3072, 768)]
    # uniform sizes reproduce the tile_T plan
    for T in (0, 64, 256):
        a = mm.plan_query(shapes, K=5, tile_T=T)
        b = mm.plan_query(shapes, K=5, tile_sizes=[T] * 4)
        assert a == b
    # mixed: full, resident 128, GEMM-engine 256, resident 96 (ragged)
    q = mm.plan_query(shapes, K=5, tile_sizes=[0, 128, 256, 96])
    assert q["units"] == 1 + 36 + 36 + 32 * 8
    each = [mm.plan_query([sh], K=5, tile_T=T)["ns_flops"] for sh, T in zip(shapes, [0, 128, 256, 96])]
    assert abs(q["ns_flops"] - sum(each)) <= 4


def test_per_matrix_tile_sizes_validation():
    with pytest.raises(mm.MuonhError):
        mm.plan_query([(64, 64), (64, 64)], K=5, tile_sizes=[0, 200])  # 200: not a multiple of 64 above 128
    with pytest.raises(ValueError):
        mm.plan_query([(64, 64), (64, 64)], K=5, tile_sizes=[64])


def test_plan_query_32bit_operand_offset_limit():
    # The GEMM engine addresses an operand buffer with 32-bit byte offsets:
    # (pad256(longer side) * pad64(shorter side) + 256) * operand bytes must
    # stay below 4 GiB.  bf16: 32704 x 65536 is the largest side pair at
    # 65536 rows of X^T (65536 * 32704 * 2 + 512 < 2^32); 32768 x 65536 is not.
    q = mm.plan_query([(32704, 65536)], K=5, workspace_limit=1 << 40)
    assert q["units"] == 1
    with pytest.raises(mm.MuonhError) as e:
        mm.plan_query([(32768, 65536)], K=5, workspace_limit=1 << 40)
    assert e.value.code == mm.MUONH_ENOTIMPL
    # the longer side counts padded to 256 rows: 65409 pads to 65472 at 64
    # (which would fit) but to 65536 at 256
    with pytest.raises(mm.MuonhError):
        mm.plan_query([(32768, 65409)], K=5, workspace_limit=1 << 40)


def test_noalloc_step_rejects_oversize_before_any_gpu_call():
    # 8192 x 8192 full-matrix Newton-Schulz needs far more than the static
    # scratch: rejected on the host, no HIP call (this machine has no GPU)
    lib = mm.load()
    P = ctypes.c_void_p * 1
    ps, gs, ms = P(0x1000), P(0x2000), P(0x3000)
    sh = (ctypes.c_int64 * 2)(8192, 8192)
    rh = (ctypes.c_float * 1)(1.0)
    o = _opts()
    rc = lib.muonh_step_noalloc(ps, gs, ms, sh, 1, 0.02, 0.95, 5, rh, 0, ctypes.byref(o))
    assert rc == mm.MUONH_ENOMEM
    assert "scratch" in lib.muonh_last_error().decode()
    # invalid arguments are rejected as by muonh_step
    assert lib.muonh_step_noalloc(ps, gs, ms, sh, 0, 0.02, 0.95, 5, rh, 0, ctypes.byref(o)) == mm.MUONH_EINVAL
    assert lib.muonh_step_noalloc(ps, gs, ms, sh, 1, 0.02, 1.5, 5, rh, 0, ctypes.byref(o)) == mm.MUONH_EINVAL
