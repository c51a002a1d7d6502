"""Python binding of libmuonh: the MuonH / Hierarchical-Muon optimizer step on
AMD Instinct MI355X (gfx950).

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of ``libmuonh.so``; PyTorch supplies device memory and the current
stream.  There is no CPU fallback: if the library is not built, every entry
point raises ``MuonhUnavailable``.

Entry points mirror the C ABI in ``include/muonh.h``:

* ``muonh_step(params, grads, moms, eta, beta, K, rho, tile_T=0, noalloc=False, **opts)``
  (``noalloc=True``: ``muonh_step_noalloc``)
* ``adamh_step(params, grads, exp_avg, exp_avg_sq, eta, step, beta1, beta2, eps, rho, **opts)``
* ``ns_orthogonalize(inputs, outputs=None, K=5, tile_T=0, **opts)``
* ``frob_project(W, U, eta, rho, **opts)``
* ``get_flags()``, ``reset_flags()``, ``release()``, ``plan_query(...)``,
  ``profile_begin()``, ``profile_read()``, ``strerror(code)``, ``version()``

``opts`` keywords: ``ns_dtype`` ("bf16" | "f32"), ``ns_precision``
("h16" | "fold" | "x32"; default "h16"), ``coeffs`` (K rows of (a, b, c)), ``ns_eps``,
``zero_rel_eps``, ``hook`` ("hyperball" | "radial_brake" | "relative" | "none"),
``hyperball_step`` ("unit" | "radius"), ``tile_sizes`` (per-matrix tile sides, 0 = full),
``outward``, ``inward``, ``rb_eps``, ``workspace_limit`` (bytes),
``momentum`` ("sum" | "ema"), ``nesterov`` (bool), ``weight_decay`` (for
hook "none"), ``lanes`` (concurrent lanes 1..4; 0: library default),
``stream`` (a torch.cuda.Stream; default: the current stream).
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char, c_double, c_float, c_int, c_int64, c_size_t, c_uint64, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmuonh.so")

MUONH_OK, MUONH_EINVAL, MUONH_ENOMEM, MUONH_EHIP, MUONH_ENOTIMPL = 0, -1, -2, -3, -4
MUONH_F32, MUONH_BF16 = 0, 1
MUONH_NS_FOLD, MUONH_NS_X32, MUONH_NS_H16 = 0, 1, 2
_NS_PRECISION = {"fold": MUONH_NS_FOLD, "x32": MUONH_NS_X32, "h16": MUONH_NS_H16}
MUONH_HOOK_HYPERBALL, MUONH_HOOK_RADIAL_BRAKE, MUONH_HOOK_NONE, MUONH_HOOK_RELATIVE = 0, 1, 2, 3
MUONH_HB_STEP_UNIT, MUONH_HB_STEP_RADIUS = 0, 1

EXPORTED = (
    "muonh_default_opts", "muonh_step", "muonh_step_noalloc", "adamh_step", "ns_orthogonalize", "frob_project", "muonh_get_flags",
    "muonh_reset_flags", "muonh_strerror", "muonh_release", "muonh_plan_query",
    "muonh_profile_begin", "muonh_profile_read", "muonh_version", "muonh_last_error",
)


class MuonhUnavailable(RuntimeError):
    """libmuonh.so is missing or could not be loaded."""


class MuonhError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = f"{where}: {strerror(code) if _LIB else code} (code {code})"
        if code == MUONH_EHIP and _LIB is not None:
            msg += f" [{_LIB.muonh_last_error().decode()}]"
        super().__init__(msg)


class Opts(ctypes.Structure):
    _fields_ = [
        ("stream", c_void_p),
        ("state_dtype", c_int),
        ("ns_dtype", c_int),
        ("ns_precision", c_int),
        ("coeffs", POINTER(c_float)),
        ("ns_eps", c_float),
        ("zero_rel_eps", c_float),
        ("hook", c_int),
        ("outward", c_float),
        ("inward", c_float),
        ("rb_eps", c_float),
        ("workspace_limit", c_size_t),
        ("momentum_ema", c_int),
        ("nesterov", c_int),
        ("weight_decay", c_float),
        ("lanes", c_int),
        ("hyperball_step", c_int),
        ("tile_sizes", POINTER(c_int)),
        ("param_dtype", c_int),
        ("deterministic", c_int),
    ]


class KernelStat(ctypes.Structure):
    _fields_ = [
        ("name", c_char * 40),
        ("launches", c_uint64),
        ("total_ms", c_double),
        ("flops", c_double),
        ("bytes", c_double),
    ]


_LIB = None


def load(path: str = LIB_PATH):
    """Load libmuonh.so (once) and declare its signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise MuonhUnavailable(
            f"{path} is not built; run `python -m matrix_orthogonalizing_optimizer_momentum_amd.build`")
    # The library must share PyTorch's HIP runtime (device pointers and
    # streams come from it): load torch first so that its libamdhip64 is the
    # one the dynamic linker binds, instead of a second runtime instance.
    try:
        import torch  # noqa: F401
    except ImportError:  # pragma: no cover - torch is only needed for tensors
        pass
    try:
        lib = ctypes.CDLL(path)
    except OSError as e:  # pragma: no cover
        raise MuonhUnavailable(f"cannot load {path}: {e}") from e
    pp = POINTER(c_void_p)
    lib.muonh_default_opts.argtypes = [POINTER(Opts)]
    lib.muonh_default_opts.restype = None
    lib.muonh_step.argtypes = [pp, pp, pp, POINTER(c_int64), c_int, c_float, c_float, c_int,
                               POINTER(c_float), c_int, POINTER(Opts)]
    lib.muonh_step.restype = c_int
    lib.muonh_step_noalloc.argtypes = lib.muonh_step.argtypes
    lib.muonh_step_noalloc.restype = c_int
    lib.adamh_step.argtypes = [pp, pp, pp, pp, POINTER(c_int64), c_int, c_float, c_float, c_float, c_float,
                               c_int64, POINTER(c_float), POINTER(Opts)]
    lib.adamh_step.restype = c_int
    lib.ns_orthogonalize.argtypes = [pp, pp, POINTER(c_int64), c_int, c_int, c_int, POINTER(Opts)]
    lib.ns_orthogonalize.restype = c_int
    lib.frob_project.argtypes = [pp, pp, POINTER(c_int64), c_int, c_float, POINTER(c_float), POINTER(Opts)]
    lib.frob_project.restype = c_int
    lib.muonh_get_flags.argtypes = [POINTER(c_uint64)]
    lib.muonh_get_flags.restype = c_int
    lib.muonh_reset_flags.argtypes = []
    lib.muonh_reset_flags.restype = c_int
    lib.muonh_strerror.argtypes = [c_int]
    lib.muonh_strerror.restype = ctypes.c_char_p
    lib.muonh_release.argtypes = []
    lib.muonh_release.restype = None
    lib.muonh_plan_query.argtypes = [POINTER(c_int64), c_int, c_int, c_int, POINTER(Opts), c_size_t,
                                     POINTER(c_int64)]
    lib.muonh_plan_query.restype = c_int
    lib.muonh_profile_begin.argtypes = []
    lib.muonh_profile_begin.restype = c_int
    lib.muonh_profile_read.argtypes = [POINTER(KernelStat), c_int, POINTER(c_int)]
    lib.muonh_profile_read.restype = c_int
    lib.muonh_version.argtypes = []
    lib.muonh_version.restype = ctypes.c_char_p
    lib.muonh_last_error.argtypes = []
    lib.muonh_last_error.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def available() -> bool:
    try:
        load()
        return True
    except MuonhUnavailable:
        return False


def strerror(code: int) -> str:
    return load().muonh_strerror(int(code)).decode()


def version() -> str:
    return load().muonh_version().decode()


def _check(rc: int, where: str):
    if rc != MUONH_OK:
        raise MuonhError(rc, where)


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------

def _check_tile_sizes(opts, n):
    ts = opts.get("tile_sizes")
    if ts is not None and len(ts) != n:
        raise ValueError(f"tile_sizes needs one entry per matrix ({n}), got {len(ts)}")


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return MUONH_BF16
    if t.dtype == torch.float32:
        return MUONH_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use torch.bfloat16 or torch.float32")


def make_opts(state_dtype=MUONH_BF16, ns_dtype="bf16", ns_precision="h16", coeffs=None, ns_eps=None,
              zero_rel_eps=None, hook="hyperball", outward=None, inward=None, rb_eps=None,
              workspace_limit=0, stream=None, K=None, momentum="sum", nesterov=False, weight_decay=None, lanes=0,
              hyperball_step="unit", tile_sizes=None):
    """Build an Opts struct; returns (opts, keepalive) where keepalive holds
    buffers the struct points to."""
    lib = load()
    o = Opts()
    lib.muonh_default_opts(ctypes.byref(o))
    o.state_dtype = state_dtype
    o.ns_dtype = {"bf16": MUONH_BF16, "f32": MUONH_F32}[ns_dtype]
    o.ns_precision = _NS_PRECISION[ns_precision]
    keep = []
    if coeffs is not None:
        flat = [float(v) for row in coeffs for v in row]
        if K is not None and len(flat) < 3 * K:
            raise ValueError("coefficient table shorter than K")
        arr = (c_float * len(flat))(*flat)
        keep.append(arr)
        o.coeffs = ctypes.cast(arr, POINTER(c_float))
    if ns_eps is not None:
        o.ns_eps = ns_eps
    if zero_rel_eps is not None:
        o.zero_rel_eps = zero_rel_eps
    o.hook = {"hyperball": MUONH_HOOK_HYPERBALL, "radial_brake": MUONH_HOOK_RADIAL_BRAKE,
              "none": MUONH_HOOK_NONE, "relative": MUONH_HOOK_RELATIVE}[hook]
    o.hyperball_step = {"unit": MUONH_HB_STEP_UNIT, "radius": MUONH_HB_STEP_RADIUS}[hyperball_step]
    if tile_sizes is not None:
        ts = (c_int * len(tile_sizes))(*[int(v) for v in tile_sizes])
        keep.append(ts)
        o.tile_sizes = ctypes.cast(ts, POINTER(c_int))
    o.momentum_ema = {"sum": 0, "ema": 1}[momentum]
    o.nesterov = 1 if nesterov else 0
    if weight_decay is not None:
        o.weight_decay = weight_decay
    o.lanes = int(lanes)
    if outward is not None:
        o.outward = outward
    if inward is not None:
        o.inward = inward
    if rb_eps is not None:
        o.rb_eps = rb_eps
    o.workspace_limit = int(workspace_limit)
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    o.stream = c_void_p(int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream))
    return o, keep


def _ptrs(ts):
    return (c_void_p * len(ts))(*[c_void_p(t.data_ptr()) if t is not None else None for t in ts])


def _shapes(ts):
    flat = []
    for t in ts:
        if t.dim() != 2:
            raise ValueError("every tensor must be a matrix (2-D)")
        flat += [int(t.shape[0]), int(t.shape[1])]
    return (c_int64 * len(flat))(*flat)


def _check_dev(ts, what):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{what}: tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError(f"{what}: tensors must be contiguous")


# --------------------------------------------------------------------------
# entry points
# --------------------------------------------------------------------------

def muonh_step(params, grads, moms, eta, beta, K, rho=None, tile_T=0, noalloc=False, **opts):
    """One MuonH step in place on ``params`` (fp32) and ``moms``.  With
    ``noalloc`` the call goes to ``muonh_step_noalloc`` (no device allocation:
    the library's static scratch; see the header for its limit)."""
    import torch
    lib = load()
    n = len(params)
    if not (len(grads) == n and len(moms) == n) or n == 0:
        raise ValueError("params, grads and moms must be non-empty lists of equal length")
    _check_dev(params, "params"); _check_dev(grads, "grads"); _check_dev(moms, "moms")
    for p, g, m in zip(params, grads, moms):
        if p.dtype != torch.float32:
            raise TypeError("params must be float32 master weights")
        if p.shape != g.shape or p.shape != m.shape:
            raise ValueError("param, grad and momentum shapes differ")
        if g.dtype != m.dtype:
            raise TypeError("grads and moms must share a dtype")
    sd = _dtype_code(grads[0])
    if any(_dtype_code(g) != sd for g in grads):
        raise TypeError("all grads must share a dtype")
    _check_tile_sizes(opts, n)
    o, keep = make_opts(state_dtype=sd, K=K, **opts)
    rho_arr = (c_float * n)(*[float(r) for r in rho]) if rho is not None else None
    fn = lib.muonh_step_noalloc if noalloc else lib.muonh_step
    rc = fn(_ptrs(params), _ptrs(grads), _ptrs(moms), _shapes(params), n, float(eta), float(beta),
            int(K), rho_arr, int(tile_T), ctypes.byref(o))
    _check(rc, "muonh_step_noalloc" if noalloc else "muonh_step")


def adamh_step(params, grads, exp_avg, exp_avg_sq, eta, step, beta1=0.9, beta2=0.95, eps=1e-8, rho=None,
               **opts):
    """One AdamH step (Hyperball around Adam's update; ``hook="none"``: AdamW)
    in place on ``params`` (fp32) and the fp32 moments; ``step`` is 1-based."""
    import torch
    lib = load()
    n = len(params)
    if not (len(grads) == n and len(exp_avg) == n and len(exp_avg_sq) == n) or n == 0:
        raise ValueError("params, grads and moments must be non-empty lists of equal length")
    for name, ts in (("params", params), ("grads", grads), ("exp_avg", exp_avg), ("exp_avg_sq", exp_avg_sq)):
        _check_dev(ts, name)
    for p, g, m, v in zip(params, grads, exp_avg, exp_avg_sq):
        if p.dtype != torch.float32 or m.dtype != torch.float32 or v.dtype != torch.float32:
            raise TypeError("params and Adam moments must be float32")
        if not (p.shape == g.shape == m.shape == v.shape):
            raise ValueError("param, grad and moment shapes differ")
    sd = _dtype_code(grads[0])
    if any(_dtype_code(g) != sd for g in grads):
        raise TypeError("all grads must share a dtype")
    o, keep = make_opts(state_dtype=sd, **opts)
    rho_arr = (c_float * n)(*[float(r) for r in rho]) if rho is not None else None
    rc = lib.adamh_step(_ptrs(params), _ptrs(grads), _ptrs(exp_avg), _ptrs(exp_avg_sq), _shapes(params), n,
                        float(eta), float(beta1), float(beta2), float(eps), int(step), rho_arr, ctypes.byref(o))
    _check(rc, "adamh_step")


def ns_orthogonalize(inputs, outputs=None, K=5, tile_T=0, **opts):
    """outputs[i] = NS_K(inputs[i]) (tiled when tile_T > 0); returns outputs."""
    import torch
    lib = load()
    n = len(inputs)
    if n == 0:
        raise ValueError("no inputs")
    if outputs is None:
        outputs = [torch.empty_like(x) for x in inputs]
    _check_dev(inputs, "inputs"); _check_dev(outputs, "outputs")
    sd = _dtype_code(inputs[0])
    for x, y in zip(inputs, outputs):
        if x.shape != y.shape or _dtype_code(x) != sd or _dtype_code(y) != sd:
            raise ValueError("inputs and outputs must match in shape and share one dtype")
    _check_tile_sizes(opts, n)
    o, keep = make_opts(state_dtype=sd, K=K, **opts)
    rc = lib.ns_orthogonalize(_ptrs(inputs), _ptrs(outputs), _shapes(inputs), n, int(K), int(tile_T),
                              ctypes.byref(o))
    _check(rc, "ns_orthogonalize")
    return outputs


def frob_project(W, U, eta, rho, **opts):
    """W[i] <- rho[i] * Pi(W[i] - eta * U[i] / ||U[i]||) in place (U=None: plain projection)."""
    import torch
    lib = load()
    n = len(W)
    _check_dev(W, "W")
    for w in W:
        if w.dtype != torch.float32:
            raise TypeError("W must be float32")
    sd = MUONH_BF16
    uptr = None
    if U is not None:
        _check_dev(U, "U")
        us = [u for u in U if u is not None]
        if us:
            sd = _dtype_code(us[0])
        uptr = _ptrs(U)
    o, keep = make_opts(state_dtype=sd, **opts)
    rho_arr = (c_float * n)(*[float(r) for r in rho])
    rc = lib.frob_project(_ptrs(W), uptr, _shapes(W), n, float(eta), rho_arr, ctypes.byref(o))
    _check(rc, "frob_project")


def get_flags():
    """(zero_update, restored, unrestorable, nonfinite) counters; synchronizes."""
    out = (c_uint64 * 4)()
    _check(load().muonh_get_flags(out), "muonh_get_flags")
    return tuple(int(v) for v in out)


def reset_flags():
    _check(load().muonh_reset_flags(), "muonh_reset_flags")


def release():
    load().muonh_release()


def plan_query(shapes, K=5, tile_T=0, workspace_limit=0, **opts):
    """Host-only planning query: dict(chunks, ws_bytes, units, ns_flops, jobs_per_iter, stream_bytes, lanes)."""
    lib = load()
    flat = [int(v) for hw in shapes for v in hw]
    arr = (c_int64 * len(flat))(*flat)
    o = Opts()
    lib.muonh_default_opts(ctypes.byref(o))
    if "ns_dtype" in opts:
        o.ns_dtype = {"bf16": MUONH_BF16, "f32": MUONH_F32}[opts["ns_dtype"]]
    if "ns_precision" in opts:
        o.ns_precision = _NS_PRECISION[opts["ns_precision"]]
    if "lanes" in opts:
        o.lanes = int(opts["lanes"])
    keep = []
    if opts.get("tile_sizes") is not None:
        _check_tile_sizes(opts, len(shapes))
        ts = (c_int * len(shapes))(*[int(v) for v in opts["tile_sizes"]])
        keep.append(ts)
        o.tile_sizes = ctypes.cast(ts, POINTER(c_int))
    if "state_dtype" in opts:
        o.state_dtype = {"bf16": MUONH_BF16, "f32": MUONH_F32}[opts["state_dtype"]]
    out = (c_int64 * 7)()
    rc = lib.muonh_plan_query(arr, len(shapes), int(K), int(tile_T), ctypes.byref(o), int(workspace_limit), out)
    _check(rc, "muonh_plan_query")
    keys = ("chunks", "ws_bytes", "units", "ns_flops", "jobs_per_iter", "stream_bytes", "lanes")
    return dict(zip(keys, (int(v) for v in out)))


def profile_begin():
    _check(load().muonh_profile_begin(), "muonh_profile_begin")


def profile_read():
    """{kernel class: dict(launches, total_ms, avg_ms, flops, bytes)} since profile_begin()."""
    lib = load()
    buf = (KernelStat * 16)()
    n = c_int(0)
    _check(lib.muonh_profile_read(buf, 16, ctypes.byref(n)), "muonh_profile_read")
    out = {}
    for i in range(n.value):
        s = buf[i]
        out[s.name.decode()] = dict(launches=int(s.launches), total_ms=s.total_ms,
                                    avg_ms=s.total_ms / max(1, s.launches), flops=s.flops, bytes=s.bytes)
    return out
