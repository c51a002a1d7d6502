"""Benchmark of one MuonH optimizer step on one MI355X.

Default workload: the GPT-2-small matrix set (12 layers x {768x2304 qkv,
768x768 attn-out, 768x3072 fc, 3072x768 proj} = 48 matrices), bf16 gradients
and momentum, fp32 master weights, K = 5 quintic Newton-Schulz iterations on
the full matrices, Hyperball with rho = ||W0||_F.  Gradients are Gaussian
(sigma = 1e-3) plus a rank-4 spike of 10x entrywise magnitude, drawn on the
device from a fixed seed; several gradient sets are pre-generated and used in
turn, so the timed region only runs optimizer steps on HBM-resident data.

One step = momentum, Newton-Schulz, Hyperball for all 48 matrices (the whole
hot path).  Timing: W untimed steps, then exactly K timed steps between two
device synchronizations, with the library's lanes (concurrent streams) as
chosen by --lanes.  A second pass of the same K steps records a HIP event
pair around every kernel launch (on the stream it runs on) to get the
per-kernel average durations behind the roofline figures; it runs with
--profile-lanes (default 1: no concurrent lanes, so a launch's duration is
its own).  The headline value comes from the first, event-free pass.

    python bench.py [--steps K] [--warmup W] [--workload gpt2|qwen1p2b|dense8b|single256]
                    [--tile T] [--ns-precision x32|fold] [--lanes L] [--profile-lanes L]
                    [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MuonH optimizer steps/sec + NS TFLOP/s (% bf16 MFMA peak), HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3     # dense fp32 MFMA
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0

NS_CLASSES = ("ns_gram_G1", "ns_poly_G2", "ns_update_G3", "ns_tile_resident")
STREAM_CLASSES = ("momentum_prep", "hook_reduce", "hook_write", "adam_moments", "adam_write")


def measured_traffic(cls, args):
    """HBM bytes per launch of kernel class ``cls`` from the committed counter
    summary (FETCH_SIZE / WRITE_SIZE runs, scaled by a plain-copy
    calibration), or None when this run's workload differs from the profiled
    one or the kernel sources changed since the counters were taken."""
    import glob
    import hashlib
    path = os.path.join(ROOT, "profiles", "muonh_step_gpt2_small_hbm_traffic.json")
    if (args.workload, args.tile, args.K, args.ns_precision, args.ws_limit_mib, args.profile_lanes) != \
            ("gpt2", 0, 5, "fold", 0, 1):
        return None
    if not os.path.exists(path):
        return None
    with open(path) as f:
        doc = json.load(f)
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "matrix_orthogonalizing_optimizer_momentum_amd", "csrc", "*"))):
        h.update(os.path.basename(p).encode())
        with open(p, "rb") as f:
            h.update(f.read())
    if h.hexdigest() != doc.get("csrc_sha256"):
        return None
    k = doc.get("kernels", {}).get(cls)
    return k["hbm_bytes_per_launch"] if k else None


HOOK_DESC = {
    "hyperball": "Hyperball rho=||W0||_F",
    "radial_brake": "RadialBrake (outward 0.5, inward 1.0, eta 0.02)",
    "relative": "RelativeUpdate (step eta*||W||_F along O/||O||_F)",
    "none": "Muon's own update (shape-scaled O, no weight decay)",
}


def workload_shapes(name):
    from synth import gen
    if name == "gpt2":
        return gen.gpt2_small_shapes(), "gpt2-small matrix set: 12 x {768x2304, 768x768, 768x3072, 3072x768}"
    if name == "qwen1p2b":
        return gen.qwen3_1p2b_shapes(), "qwen3-style 1.2B matrix set: 28 x {2048x2048 q, 2048x1024 k, 2048x1024 v, 2048x2048 o, 2048x6144 gate, 2048x6144 up, 6144x2048 down}"
    if name == "dense8b":
        return gen.dense_8b_shapes(), "8B-shaped dense matrix set: 32 x {4096x4096 q, 4096x1024 k, 4096x1024 v, 4096x4096 o, 4096x14336 gate, 4096x14336 up, 14336x4096 down}"
    if name == "single256":
        return [(256, 256)], "single 256x256 matrix"
    if name == "single64x128":
        return [(64, 128)], "single 64x128 matrix"
    raise SystemExit(f"unknown workload {name}")


def make_device_inputs(shapes, nsets, seed, torch, state_dtype=None):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    Ws, Ms, Gsets = [], [], []
    for H, W in shapes:
        Ws.append((torch.randn(H, W, generator=g, device="cuda") * 0.02).contiguous())
        Ms.append(torch.zeros(H, W, device="cuda", dtype=state_dtype or torch.bfloat16))
    sigma, rank, mag = 1e-3, 4, 10.0
    for _ in range(nsets):
        gs = []
        for H, W in shapes:
            Z = torch.randn(H, W, generator=g, device="cuda")
            A = torch.randn(H, rank, generator=g, device="cuda")
            B = torch.randn(W, rank, generator=g, device="cuda")
            G = sigma * Z + (mag * sigma / math.sqrt(rank)) * (A @ B.t())
            gs.append(G.to(state_dtype or torch.bfloat16).contiguous())
        Gsets.append(gs)
    rho = [float(torch.linalg.vector_norm(w.double())) for w in Ws]
    return Ws, Ms, Gsets, rho


def _ns_flops(H, W, K, T):
    def full(h, w):
        r, q = min(h, w), max(h, w)
        return K * (4.0 * r * r * q + 2.0 * r ** 3)
    if T <= 0:
        return full(H, W)
    return sum(full(min(T, H - a), min(T, W - b)) for a in range(0, H, T) for b in range(0, W, T))


def cpu_baseline(shapes, K, tile_T, hook, budget_s=12.0):
    """The fp64 numpy oracle, as it stands, on a bounded sample of the same
    workload: whole matrices in the workload's order until ~budget_s of CPU
    time; when the set is not finished, the time is extrapolated to the full
    set by its share of the Newton-Schulz flops (which dominate the oracle)."""
    import numpy as np
    from oracle import muonh_oracle as orc
    from synth import gen
    try:
        from threadpoolctl import threadpool_info
        cores = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    total_f = sum(_ns_flops(h, w, K, tile_T) for h, w in shapes)
    total_e = sum(h * w for h, w in shapes)
    t_sum, t_ns, f_sum, e_sum, done = 0.0, 0.0, 0.0, 0, 0
    t_all = time.perf_counter()
    while done < len(shapes) and (time.perf_counter() - t_all) < budget_s:
        sub = [shapes[done]]
        Ws, Gs, Ms = gen.model_set(sub, 2, 1)
        rho = [float(np.linalg.norm(w.astype(np.float64))) for w in Ws]
        t0 = time.perf_counter()
        orc.muonh_step(Ws, Gs, Ms, 0.02, 0.95, K, rho, tile_T=tile_T, hook=hook, state_bf16=True)
        t_sum += time.perf_counter() - t0
        # its Newton-Schulz phase on its own (zero momentum: the NS input is G)
        t0 = time.perf_counter()
        orc.orthogonalize(Gs[0], K, tile_T)
        t_ns += time.perf_counter() - t0
        f_sum += _ns_flops(sub[0][0], sub[0][1], K, tile_T)
        e_sum += sub[0][0] * sub[0][1]
        done += 1
    whole = done == len(shapes)
    ns_s = t_ns if whole else t_ns * total_f / f_sum
    stream_s = max(t_sum - t_ns, 0.0) * (1.0 if whole else total_e / e_sum)
    step_s = t_sum if whole else ns_s + stream_s
    how = ("the whole set" if whole else
           f"extrapolated to the full set by its Newton-Schulz flops and elements ({f_sum / total_f:.2%} "
           f"of the flops sampled)")
    return {"value": 1.0 / step_s, "unit": "steps/s", "cores": cores, "kind": "oracle",
            "ns_s_per_step": round(ns_s, 4), "stream_s_per_step": round(stream_s, 4),
            "sample": f"{done} of {len(shapes)} matrices timed with the fp64 numpy oracle, {t_sum:.1f} s "
                      f"(Newton-Schulz timed again on its own, {t_ns:.1f} s); {how}: {step_s:.1f} s/step"}


def cpu_baseline_adamh(shapes, hook, budget_s=12.0):
    """The fp64 oracle's AdamH step on the same matrix set (streaming only,
    so the whole set fits the budget on the host's cores; else extrapolated by
    element count)."""
    import numpy as np
    from oracle import muonh_oracle as orc
    from synth import gen
    try:
        from threadpoolctl import threadpool_info
        cores = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    total = sum(h * w for h, w in shapes)
    t_sum, e_sum, done = 0.0, 0, 0
    t_all = time.perf_counter()
    while done < len(shapes) and (time.perf_counter() - t_all) < budget_s:
        sub = [shapes[done]]
        Ws, Gs, _ = gen.model_set(sub, 2, 1)
        Z = [np.zeros(s) for s in sub]
        rho = [float(np.linalg.norm(w.astype(np.float64))) for w in Ws]
        t0 = time.perf_counter()
        orc.adamh_step(Ws, Gs, Z, Z, 0.02, 0.9, 0.95, 1e-8, 1, rho, hook=hook)
        t_sum += time.perf_counter() - t0
        e_sum += sub[0][0] * sub[0][1]
        done += 1
    step_s = t_sum if done == len(shapes) else t_sum * total / e_sum
    return {"value": 1.0 / step_s, "unit": "steps/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} of {len(shapes)} matrices timed with the fp64 numpy oracle's AdamH step, "
                      f"{t_sum:.1f} s; {step_s:.2f} s/step"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gpt2")
    ap.add_argument("--tile", type=int, default=0)
    ap.add_argument("--ns-precision", default="fold", choices=["fold", "x32"])
    ap.add_argument("--hook", default="hyperball", choices=["hyperball", "radial_brake", "relative", "none"])
    ap.add_argument("--optimizer", default="muonh", choices=["muonh", "adamh"],
                    help="adamh: the Hyperball wrapper around Adam (streaming only, no Newton-Schulz)")
    ap.add_argument("--K", type=int, default=5)
    ap.add_argument("--lanes", type=int, default=0, choices=[0, 1, 2, 3, 4],
                    help="concurrent lanes of a timed step (0: the library's automatic choice)")
    ap.add_argument("--profile-lanes", type=int, default=1, choices=[0, 1, 2, 3, 4],
                    help="lanes of the per-launch timing pass (1: every launch has the GPU to itself)")
    ap.add_argument("--state", default="bf16", choices=["bf16", "f32"],
                    help="gradient and momentum storage type (f32: the all-fp32 single-matrix setting)")
    ap.add_argument("--ns-dtype", default="bf16", choices=["bf16", "f32"],
                    help="Newton-Schulz operand type (f32 runs on fp32 MFMA)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of HIP graphs that captured one whole step per gradient set "
                         "(after the warm-up has planned the call, so the captured launches allocate nothing)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--grad-sets", type=int, default=4)
    ap.add_argument("--ws-limit-mib", type=int, default=0,
                    help="workspace limit (MiB): matrices run in chunks that fit it; 0 = library default")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="run a plain device copy of this many MiB first (counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU's share of the step: this build runs on a single GPU "
              "(no collectives); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import matrix_orthogonalizing_optimizer_momentum_amd as mm
    if not os.path.exists(mm.LIB_PATH):
        from matrix_orthogonalizing_optimizer_momentum_amd import build as b
        b.build()
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    shapes, wdesc = workload_shapes(args.workload)
    K = args.K
    Ws, Ms, Gsets, rho = make_device_inputs(shapes, args.grad_sets, 1234, torch,
                                            torch.float32 if args.state == "f32" else torch.bfloat16)
    ns_peak = PEAK_BF16_TFLOPS if args.ns_dtype == "bf16" else PEAK_F32_TFLOPS
    ws_limit = args.ws_limit_mib << 20
    q = mm.plan_query(shapes, K=K, tile_T=args.tile, ns_precision=args.ns_precision, workspace_limit=ws_limit,
                      ns_dtype=args.ns_dtype, lanes=args.lanes)
    qb = mm.plan_query(shapes, K=K, tile_T=args.tile, ns_precision=args.ns_precision, workspace_limit=ws_limit,
                       ns_dtype=args.ns_dtype, lanes=args.profile_lanes)
    if args.copy_calib_mib:
        # a plain copy kernel of known size: reads and writes copy_calib_mib MiB each
        n = args.copy_calib_mib * (1 << 20) // 4
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        del src, dst
    torch.cuda.synchronize()

    if args.optimizer == "adamh":
        Ms = [torch.zeros(w.shape, device="cuda") for w in Ws]  # fp32 Adam moments
        Vs = [torch.zeros(w.shape, device="cuda") for w in Ws]
    counter = [0]

    def step(i, lanes=args.lanes):
        if args.optimizer == "adamh":
            counter[0] += 1
            mm.adamh_step(Ws, Gsets[i % len(Gsets)], Ms, Vs, 0.02, counter[0], rho=rho, hook=args.hook,
                          workspace_limit=ws_limit)
            return
        mm.muonh_step(Ws, Gsets[i % len(Gsets)], Ms, eta=0.02, beta=0.95, K=K, rho=rho, tile_T=args.tile,
                      ns_dtype=args.ns_dtype,
                      lanes=lanes,
                      ns_precision=args.ns_precision, workspace_limit=ws_limit, hook=args.hook)

    for i in range(max(args.warmup, len(Gsets) if args.graph else 0)):
        step(i)
    torch.cuda.synchronize()
    run = step
    if args.graph:
        # one graph per gradient set, each the whole step on the same buffers
        graphs = []
        for k in range(len(Gsets)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(k)
            graphs.append(g)
        torch.cuda.synchronize()

        def run(i):
            graphs[i % len(graphs)].replay()

    # pass A: headline, no events
    t0 = time.perf_counter()
    for i in range(args.steps):
        run(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    # pass B: same steps with per-launch HIP events.  By default the lanes are
    # off here, so each launch's duration is its own and not shared with a
    # concurrent lane's kernels.
    for i in range(2):
        step(i, args.profile_lanes)
    torch.cuda.synchronize()
    mm.profile_begin()
    tb0 = time.perf_counter()
    for i in range(args.steps):
        step(i, args.profile_lanes)
    torch.cuda.synchronize()
    tb1 = time.perf_counter()
    prof = mm.profile_read()
    ms_b = (tb1 - tb0) * 1e3 / args.steps

    ns_ms = sum(prof[c]["total_ms"] for c in NS_CLASSES if c in prof) / args.steps
    st_ms = sum(prof[c]["total_ms"] for c in STREAM_CLASSES if c in prof) / args.steps
    st_bytes = sum(prof[c]["bytes"] for c in STREAM_CLASSES if c in prof) / args.steps
    ns_tflops = q["ns_flops"] / (ns_ms * 1e-3) / 1e12 if ns_ms > 0 else None
    stream_gbs = st_bytes / (st_ms * 1e-3) / 1e9 if st_ms > 0 else None

    dom = max(prof, key=lambda c: prof[c]["total_ms"])
    d = prof[dom]
    # The resident-tile kernel also streams its tiles' state (read G, M and W,
    # write M and O): it is bound by whichever floor is higher, matrix-core
    # time or HBM time (HBM for T = 64 on bf16 state, about even at T = 128).
    tile_hbm = (dom == "ns_tile_resident" and d["bytes"] > 0 and
                d["bytes"] / (PEAK_HBM_GBS * 1e9) > d["flops"] / (ns_peak * 1e12))
    if dom in NS_CLASSES and not tile_hbm:
        per_launch = d["flops"] / d["launches"]
        achieved = per_launch / (d["avg_ms"] * 1e-3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2), "peak": ns_peak,
                "unit": "TFLOP/s", "frac": round(achieved / ns_peak, 4),
                "traffic": measured_traffic(dom, args),
                "flops_per_launch": per_launch, "avg_launch_ms": d["avg_ms"], "timing_lanes": qb["lanes"]}
    else:
        per_launch = d["bytes"] / d["launches"]
        achieved = per_launch / (d["avg_ms"] * 1e-3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": measured_traffic(dom, args),
                "bytes_per_launch": per_launch, "avg_launch_ms": d["avg_ms"], "timing_lanes": qb["lanes"]}

    kernels = {c: {"launches_per_step": v["launches"] / args.steps, "avg_ms": round(v["avg_ms"], 5),
                   "ms_per_step": round(v["total_ms"] / args.steps, 5)} for c, v in prof.items()}
    for c in NS_CLASSES:
        if c in prof and prof[c]["total_ms"] > 0:
            kernels[c]["tflops"] = round(prof[c]["flops"] / (prof[c]["total_ms"] * 1e-3) / 1e12, 2)
            if prof[c]["bytes"] > 0:
                kernels[c]["gbps"] = round(prof[c]["bytes"] / (prof[c]["total_ms"] * 1e-3) / 1e9, 1)
    for c in STREAM_CLASSES:
        if c in prof and prof[c]["total_ms"] > 0:
            kernels[c]["gbps"] = round(prof[c]["bytes"] / (prof[c]["total_ms"] * 1e-3) / 1e9, 1)

    if args.optimizer == "adamh":
        opt_desc = ("AdamH step (Adam betas 0.9/0.95, eps 1e-8, bias-corrected), bf16 grads, fp32 moments "
                    "and master weights, " + HOOK_DESC[args.hook])
    else:
        opt_desc = (f"MuonH step, K={K} quintic NS "
                    f"{'tiled T=' + str(args.tile) if args.tile else 'full-matrix'}, "
                    f"{args.state} grads/momentum, {args.ns_dtype} NS operands, fp32 master weights, " + HOOK_DESC[args.hook])
    out = {
        "metric": METRIC if args.optimizer == "muonh" else "AdamH optimizer steps/sec, HBM GB/s",
        "value": round(1000.0 / ms_per_step, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.ns_dtype if args.optimizer == "muonh" else "f32",
        "data": "synthetic (seeded device RNG: W0 ~ N(0, 0.02^2); grads N(0, 1e-3^2) + rank-4 10x spike)",
        "config": {"workload": f"{wdesc}; {opt_desc}", "optimizer": args.optimizer,
                   "matrices": len(shapes), "K": K, "tile_T": args.tile, "ns_precision": args.ns_precision,
                   "hook": args.hook,
                   "elements": sum(h * w for h, w in shapes),
                   "chunks": q["chunks"] if args.optimizer == "muonh" else 1,
                   "lanes": q["lanes"] if args.optimizer == "muonh" else 1,
                   "graph": bool(args.graph)},
        "ns_tflops": round(ns_tflops, 2) if ns_tflops else None,
        f"ns_frac_{args.ns_dtype}_peak": round(ns_tflops / ns_peak, 4) if ns_tflops else None,
        "ns_ms_per_step": round(ns_ms, 4),
        "stream_gbps": round(stream_gbs, 1) if stream_gbs else None,
        "stream_frac_hbm": round(stream_gbs / PEAK_HBM_GBS, 4) if stream_gbs else None,
        "stream_ms_per_step": round(st_ms, 4),
        "ms_per_step_with_events": round(ms_b, 4),
        "kernels": kernels,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = (cpu_baseline(shapes, K, args.tile, args.hook) if args.optimizer == "muonh"
                               else cpu_baseline_adamh(shapes, args.hook))
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
