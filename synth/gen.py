"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and
the benchmark.

This module holds none of the optimizer's arithmetic: it only draws numbers
(numpy PCG64 streams), rounds them to the storage dtype the workload names,
and lists the matrix shapes of the model families the pages train.

Value structure:
* weights W0 ~ N(0, 0.02^2);
* gradients G = sigma * Z + (mag * sigma / sqrt(rank)) * A B^T with Z, A, B
  i.i.d. N(0, 1), A: H x rank, B: W x rank.  The low-rank term has entrywise
  RMS mag * sigma, which gives the very high condition number the Muon
  explainer describes for transformer gradient updates (a few singular values
  dominate);
* Hadamard-built inputs for the exact-cancel case.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# storage rounding
# ---------------------------------------------------------------------------

def to_bf16_values(x) -> np.ndarray:
    """Round float values to the nearest bfloat16 (ties to even); return them
    as float32 (every value is exactly representable in bf16)."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).reshape(f.shape)


def store(x, dtype: str) -> np.ndarray:
    """Values as a tensor of ``dtype`` ("f32" or "bf16") would hold them."""
    if dtype == "bf16":
        return to_bf16_values(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).copy()
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# draws
# ---------------------------------------------------------------------------

def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(int(seed)))


def gaussian(shape, std: float, seed: int) -> np.ndarray:
    return (rng(seed).standard_normal(shape) * std).astype(np.float32)


def spiked_grad(H: int, W: int, sigma: float, seed: int, rank: int = 4, mag: float = 10.0) -> np.ndarray:
    """Gaussian gradient plus a rank-``rank`` spike of entrywise RMS mag*sigma."""
    g = rng(seed)
    Z = g.standard_normal((H, W), dtype=np.float32)
    A = g.standard_normal((H, rank), dtype=np.float32)
    B = g.standard_normal((W, rank), dtype=np.float32)
    return (sigma * Z + (mag * sigma / np.sqrt(rank)) * (A @ B.T)).astype(np.float32)


def seed_for(cfg: int, matrix: int, step: int) -> int:
    return 1_000_000 * cfg + 1_000 * matrix + step


def orthonormal(n: int, k: int, seed: int) -> np.ndarray:
    """n x k matrix with orthonormal columns (QR of a Gaussian), float64."""
    q, r = np.linalg.qr(rng(seed).standard_normal((n, k)))
    return q * np.sign(np.diag(r))


def with_singular_values(H: int, W: int, s, seed: int) -> np.ndarray:
    """U diag(s) V^T with random orthonormal U (H x k), V (W x k), float64."""
    s = np.asarray(s, dtype=np.float64)
    k = len(s)
    U = orthonormal(H, k, seed)
    V = orthonormal(W, k, seed + 1)
    return (U * s) @ V.T


def hadamard(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order n (a power of two), entries +-1."""
    if n < 1 or (n & (n - 1)):
        raise ValueError("n must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


# ---------------------------------------------------------------------------
# matrix sets (rows x cols of each weight, as stored)
# ---------------------------------------------------------------------------

def gpt2_small_shapes():
    """GPT-2 small: 12 layers x {qkv 768x2304, attn-out 768x768,
    fc 768x3072, proj 3072x768}."""
    out = []
    for _ in range(12):
        out += [(768, 2304), (768, 768), (768, 3072), (3072, 768)]
    return out


def qwen3_1p2b_shapes():
    """Qwen3-style 1.2B: 28 layers x {q 2048x2048, k 2048x1024, v 2048x1024,
    o 2048x2048, gate 2048x6144, up 2048x6144, down 6144x2048}."""
    out = []
    for _ in range(28):
        out += [(2048, 2048), (2048, 1024), (2048, 1024), (2048, 2048),
                (2048, 6144), (2048, 6144), (6144, 2048)]
    return out


def dense_8b_shapes():
    """8B-shaped dense set: 32 layers x {q 4096x4096, k 4096x1024,
    v 4096x1024, o 4096x4096, gate 4096x14336, up 4096x14336,
    down 14336x4096}."""
    out = []
    for _ in range(32):
        out += [(4096, 4096), (4096, 1024), (4096, 1024), (4096, 4096),
                (4096, 14336), (4096, 14336), (14336, 4096)]
    return out


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

def single_matrix_case(H: int, W: int, steps: int = 10, seed_w: int = 0, seed_g0: int = 1000):
    """The single-matrix fp32 case: W0, G_t ~ N(0, 0.02^2), M0 = 0."""
    W0 = gaussian((H, W), 0.02, seed_w)
    Gs = [gaussian((H, W), 0.02, seed_g0 + t) for t in range(1, steps + 1)]
    M0 = np.zeros((H, W), np.float32)
    return W0, Gs, M0


def exact_cancel_case(H: int, W: int, rho: float = 0.5, eta: float = 0.5, c: float = 1.0):
    """Inputs whose Hyperball update cancels W exactly.

    Hd is a +-1 matrix with orthogonal rows (Sylvester Hadamard, or [H H] for
    H x 2H); W0 = rho * Hd / sqrt(H*W) has norm rho, the gradient is c * Hd
    and the momentum starts at zero.  With eta = rho the orthogonalized,
    unit-normalized update equals W0 / rho, so W0 - eta * U_hat = 0.
    """
    if W == H:
        Hd = hadamard(H)
    elif W == 2 * H:
        h = hadamard(H)
        Hd = np.concatenate([h, h], axis=1)
    else:
        raise ValueError("exact-cancel case needs W == H or W == 2H")
    W0 = (rho * Hd / np.sqrt(H * W)).astype(np.float32)
    G = (c * Hd).astype(np.float32)
    M0 = np.zeros((H, W), np.float32)
    return W0, G, M0, float(rho), float(eta)


def model_set(shapes, cfg: int, step: int, sigma: float = 1e-3, state: str = "bf16"):
    """Weights, one step of spiked gradients and zero momentum for a matrix set.
    Weights are float32 master copies; grads are stored in ``state`` dtype."""
    Ws, Gs, Ms = [], [], []
    for i, (H, W) in enumerate(shapes):
        Ws.append(gaussian((H, W), 0.02, seed_for(cfg, i, 0)))
        Gs.append(store(spiked_grad(H, W, sigma, seed_for(cfg, i, step)), state))
        Ms.append(np.zeros((H, W), np.float32))
    return Ws, Gs, Ms
