"""muonh_step_noalloc (no device allocation: the library's static scratch)
against muonh_step on the same inputs, through the C ABI: two calls in a
row, the second with a smaller input; full-matrix Newton-Schulz on the GEMM
engine and resident HiMuon tiles.  The same kernels run on both paths, so
the results must be bitwise equal."""
import numpy as np
import pytest

from synth import gen

torch = pytest.importorskip("torch")
import matrix_orthogonalizing_optimizer_momentum_amd as mm  # noqa: E402

pytestmark = pytest.mark.gpu


def _inputs(shapes, seed):
    Ws, Gs, Ms = gen.model_set(shapes, 2, seed)
    Ms = [gen.store(gen.spiked_grad(H, W, 1e-3, 900 + seed + i), "bf16") for i, (H, W) in enumerate(shapes)]
    rho = [np.float32(np.linalg.norm(w.astype(np.float64))) for w in Ws]
    return Ws, Gs, Ms, rho


def _run(shapes, seed, noalloc, **kw):
    Ws, Gs, Ms, rho = _inputs(shapes, seed)
    w = [torch.from_numpy(x).cuda() for x in Ws]
    g = [torch.from_numpy(x).cuda().to(torch.bfloat16) for x in Gs]
    m = [torch.from_numpy(x).cuda().to(torch.bfloat16) for x in Ms]
    mm.muonh_step(w, g, m, eta=0.02, beta=0.95, K=5, rho=rho, noalloc=noalloc, **kw)
    torch.cuda.synchronize()
    return [t.cpu() for t in w], [t.cpu() for t in m]


@pytest.mark.parametrize("tile", [0, 64, 256])
def test_noalloc_step_matches_muonh_step_twice(tile):
    # first call: three matrices (a ragged side among them); second call: a
    # smaller single matrix, reusing the scratch the first one left behind
    calls = [[(768, 1024), (1024, 768), (300, 700)], [(256, 384)]]
    for k, shapes in enumerate(calls):
        print(f"[case] noalloc tile={tile} call {k} shapes {shapes}", flush=True)
        w_ref, m_ref = _run(shapes, 10 + k, False, tile_T=tile)
        w_na, m_na = _run(shapes, 10 + k, True, tile_T=tile)
        for i in range(len(shapes)):
            assert torch.equal(w_na[i], w_ref[i]), (k, i)
            assert torch.equal(m_na[i], m_ref[i]), (k, i)


def test_noalloc_rejects_a_call_beyond_the_scratch():
    print("[case] noalloc oversize rejected", flush=True)
    w = [torch.zeros(8192, 8192, device="cuda")]
    g = [torch.zeros(8192, 8192, device="cuda", dtype=torch.bfloat16)]
    m = [torch.zeros(8192, 8192, device="cuda", dtype=torch.bfloat16)]
    with pytest.raises(mm.MuonhError) as e:
        mm.muonh_step(w, g, m, eta=0.02, beta=0.95, K=5, rho=[1.0], noalloc=True)
    assert e.value.code == mm.MUONH_ENOMEM
    assert "scratch" in mm.load().muonh_last_error().decode()
