"""HIP graph capture of a whole optimizer step: a captured muonh_step (after
one eager call has planned it and sized the workspace) replays the same
kernels as an eager call.  Each replay is checked bit for bit against an
eager step on a second copy of the state, with the program's own eager work
and a synchronization between the replays."""
import numpy as np
import pytest

from synth import gen

torch = pytest.importorskip("torch")
import matrix_orthogonalizing_optimizer_momentum_amd as mm  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def dev(a, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.float32))).to(DEV).to(dtype).contiguous()


CASES = {
    # the all-fp32 single-matrix setting, fp32 Newton-Schulz, one lane
    "256x256-f32": dict(shapes=[(256, 256)], state=torch.float32, kw=dict(ns_dtype="f32")),
    # bf16 state on the GEMM engine, two concurrent lanes (side stream joined in the capture)
    "gemm-bf16-lanes2": dict(shapes=[(768, 768), (768, 3072), (3072, 768)], state=torch.bfloat16,
                             kw=dict(lanes=2)),
    # resident tiles (Hierarchical Muon, T = 64) with RadialBrake
    "tiles64-radial-brake": dict(shapes=[(300, 700), (256, 130)], state=torch.bfloat16,
                                 kw=dict(tile_T=64, hook="radial_brake")),
    # the fused 256-tile kernel (T = 256, ragged tiles among them)
    "tiles256-fused": dict(shapes=[(768, 768), (300, 700)], state=torch.bfloat16, kw=dict(tile_T=256)),
}


@pytest.mark.parametrize("case", list(CASES))
def test_graph_replays_match_eager_steps(case):
    c = CASES[case]
    print(f"[case] graph {case}", flush=True)
    Ws, Gs, Ms = gen.model_set(c["shapes"], 2, 1)
    rho = [np.float32(np.linalg.norm(w.astype(np.float64))) for w in Ws]
    wa = [dev(w) for w in Ws]
    ma = [dev(m, c["state"]) for m in Ms]
    g = [dev(x, c["state"]) for x in Gs]
    kw = dict(eta=0.02, beta=0.95, K=5, rho=rho, **c["kw"])
    mm.muonh_step(wa, g, ma, **kw)  # plans the call, sizes the workspace
    torch.cuda.synchronize()
    wb = [t.clone() for t in wa]
    mb = [t.clone() for t in ma]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mm.muonh_step(wa, g, ma, **kw)
    torch.cuda.synchronize()
    for rep in range(3):
        graph.replay()
        mm.muonh_step(wb, g, mb, **kw)
        torch.cuda.synchronize()
        for i in range(len(wa)):
            assert torch.equal(wa[i], wb[i]), f"replay {rep}: W[{i}] differs from the eager step"
            assert torch.equal(ma[i], mb[i]), f"replay {rep}: M[{i}] differs from the eager step"


def test_graph_survives_reduction_buffer_growth():
    # A captured step keeps the addresses of the library's reduction buffers.
    # Calls made between capture and replay that need more partial or slot
    # entries than those buffers hold (projections over many blocks and over
    # many matrices: no Newton-Schulz workspace) get larger buffers, and the
    # old ones stay allocated until muonh_release, so the replays still match
    # eager steps bit for bit.
    print("[case] graph across reduction-buffer growth", flush=True)
    mm.release()  # start from the smallest reduction buffers
    shapes = [(768, 768), (300, 700)]
    Ws, Gs, Ms = gen.model_set(shapes, 2, 3)
    rho = [np.float32(np.linalg.norm(w.astype(np.float64))) for w in Ws]
    wa = [dev(w) for w in Ws]
    ma = [dev(m, torch.bfloat16) for m in Ms]
    g = [dev(x, torch.bfloat16) for x in Gs]
    kw = dict(eta=0.02, beta=0.95, K=5, rho=rho)
    mm.muonh_step(wa, g, ma, **kw)
    torch.cuda.synchronize()
    wb = [t.clone() for t in wa]
    mb = [t.clone() for t in ma]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mm.muonh_step(wa, g, ma, **kw)
    torch.cuda.synchronize()
    # more hook blocks than the first partials buffer (8192 x 8192: 8192
    # blocks), then more matrices than its slots (1100 matrices)
    big = [torch.full((8192, 8192), 0.01, device=DEV)]
    mm.frob_project(big, None, 0.0, [float(np.sqrt(8192.0 * 8192.0) * 0.01)])
    many = [torch.full((8, 8), 0.5, device=DEV) for _ in range(1100)]
    mm.frob_project(many, None, 0.0, [4.0] * len(many))
    torch.cuda.synchronize()
    for rep in range(3):
        graph.replay()
        mm.muonh_step(wb, g, mb, **kw)
        torch.cuda.synchronize()
        for i in range(len(wa)):
            assert torch.equal(wa[i], wb[i]), f"replay {rep}: W[{i}] differs from the eager step"
            assert torch.equal(ma[i], mb[i]), f"replay {rep}: M[{i}] differs from the eager step"
    del graph
    torch.cuda.synchronize()
