"""Seeded generators for the workloads the pages describe.

Shapes follow the pages' workloads: Kimi-K2 expert matrices 2048 x 7168 (216
experts x up/gate/down), the dense 7168 x 18432 FFN weights, expert-sized
1408 x 2048 matrices, a small 128 x 512 case and a stability sweep.

Spectra: low-rank-plus-noise gradients G = U diag(s) V^T + noise * E with
s_i = i^-p, a Gaussian bulk plus a rank-32 spike, and log-uniform spectra with
random orthonormal factors. Orthonormal factors come from the QR factorisation
of a Gaussian matrix with the column signs fixed by diag(R).

Seeding: host-side matrix i of workload j uses ``numpy.random.SeedSequence([j, i])``;
device-side generation uses ``torch.Generator(device).manual_seed(10**6 * j + i)``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "host_rng", "orthonormal", "lowrank_plus_noise",
    "gaussian_plus_spike", "loguniform_spectrum", "stability_classes",
    "torch_lowrank_plus_noise", "torch_gaussian_plus_spike", "torch_weights",
    "torch_loguniform_spectrum", "structured_known_svd",
]


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    batch: int
    rows: int
    cols: int
    dtype: str


WORKLOADS = {
    "small_fp32": Workload("small_fp32", 0, 1, 128, 512, "f32"),
    "expert_1408x2048": Workload("expert_1408x2048", 1, 64, 1408, 2048, "bf16"),
    "k2_experts_648x2048x7168": Workload("k2_experts_648x2048x7168", 2, 648, 2048, 7168, "bf16"),
    "k2_dense_3x7168x18432": Workload("k2_dense_3x7168x18432", 3, 3, 7168, 18432, "bf16"),
    "stability_sweep_256": Workload("stability_sweep_256", 4, 256, 0, 0, "f16/bf16"),
}


def host_rng(workload_index: int, matrix_index: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([workload_index, matrix_index]))


def orthonormal(rng: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    """rows x cols matrix with orthonormal columns (cols <= rows), fp64."""
    A = rng.standard_normal((rows, cols))
    Q, R = np.linalg.qr(A)
    d = np.sign(np.diag(R))
    d[d == 0] = 1.0
    return Q * d


def lowrank_plus_noise(rng: np.random.Generator, rows: int, cols: int, power: float,
                       noise: float, normalize: bool = True, relative: bool = False) -> np.ndarray:
    """G = U diag(i^-power) V^T + noise * E (E ~ N(0,1) per entry), optionally scaled to
    unit Frobenius norm. relative: scale the noise term instead so that its Frobenius norm is
    noise times the signal's (keeps the power law above the noise). fp64, host side."""
    r = min(rows, cols)
    U = orthonormal(rng, rows, r)
    V = orthonormal(rng, cols, r)
    s = np.arange(1, r + 1, dtype=np.float64) ** (-power)
    E = rng.standard_normal((rows, cols))
    if relative:
        E *= np.linalg.norm(s) / np.linalg.norm(E)
    G = (U * s) @ V.T + noise * E
    if normalize:
        G = G / np.linalg.norm(G)
    return G


def gaussian_plus_spike(rng: np.random.Generator, rows: int, cols: int, rank: int = 32,
                        spike_factor: float = 10.0) -> np.ndarray:
    """E + U_r diag(sigma) V_r^T with E ~ N(0,1) per entry and sigma = spike_factor times the
    bulk edge sqrt(rows) + sqrt(cols). fp64, host side."""
    U = orthonormal(rng, rows, rank)
    V = orthonormal(rng, cols, rank)
    sigma = spike_factor * (math.sqrt(rows) + math.sqrt(cols))
    return rng.standard_normal((rows, cols)) + sigma * (U @ V.T)


def loguniform_spectrum(rng: np.random.Generator, rows: int, cols: int,
                        lo: float = 1e-6, hi: float = 1.0) -> np.ndarray:
    """U diag(s) V^T with s_j = exp(Uniform(ln lo, ln hi)) i.i.d. and random orthonormal factors."""
    r = min(rows, cols)
    U = orthonormal(rng, rows, r)
    V = orthonormal(rng, cols, r)
    s = np.exp(rng.uniform(math.log(lo), math.log(hi), size=r))
    return (U * s) @ V.T


def stability_classes(count: int = 256):
    """Shape of each matrix of the stability sweep: class c = i mod 12 selects
    n in {512, 1024, 2048}[c // 4] and n:m in {1:1, 1:2, 1:4, 1:8}[c % 4]."""
    out = []
    for i in range(count):
        c = i % 12
        n = (512, 1024, 2048)[c // 4]
        m = n * (1, 2, 4, 8)[c % 4]
        out.append((n, m))
    return out


def structured_known_svd(rng: np.random.Generator, n: int, m: int, spectrum: np.ndarray,
                         na: int, ma: int):
    """A dense n x m matrix with a known SVD, cheap at any size:
    G = (Ua kron Ub) [diag(spectrum) 0] (Va kron Vb)^T, with small random orthogonal
    Ua (na x na), Ub (n/na x n/na), Va (ma x ma), Vb (m/ma x m/ma).
    Returns (G, factors) where factors = (Ua, Ub, Va, Vb); fp64, host side.
    Entry (i, j) of U f(S) V^T is sum_t U[i, t] f(s_t) V[j, t] with U = Ua kron Ub."""
    assert n % na == 0 and m % ma == 0 and spectrum.shape == (n,)
    Ua = orthonormal(rng, na, na)
    Ub = orthonormal(rng, n // na, n // na)
    Va = orthonormal(rng, ma, ma)
    Vb = orthonormal(rng, m // ma, m // ma)
    U = np.kron(Ua, Ub)
    V = np.kron(Va, Vb)[:, :n]
    G = (U * spectrum) @ V.T
    return G, (Ua, Ub, Va, Vb)


# ---------------------------------------------------------------- device side (torch)

def _torch():
    import torch  # local import: host-only users need numpy alone
    return torch


def _tgen(device, workload_index: int, matrix_index: int):
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(10 ** 6 * workload_index + matrix_index)
    return g


def _t_orthonormal(gen, batch, rows, cols, device):
    """The Q factor (diag(R) > 0) of a Gaussian rows x cols matrix, by Cholesky QR applied
    twice in fp64: Q = A R^-1 with R^T R = A^T A. Same factor as a Householder QR with the
    signs fixed by diag(R), in a handful of batched launches."""
    torch = _torch()
    A = torch.randn(batch, rows, cols, generator=gen, device=device, dtype=torch.float32)
    A = A.to(torch.float64)
    for _ in range(2):
        L = torch.linalg.cholesky(A.transpose(-1, -2) @ A)
        A = torch.linalg.solve_triangular(L, A.transpose(-1, -2), upper=False).transpose(-1, -2)
    return A.to(torch.float32).contiguous()


def torch_lowrank_plus_noise(batch: int, rows: int, cols: int, power: float, noise: float,
                             workload_index: int, seed_offset: int = 0, device="cuda",
                             dtype=None, normalize: bool = True, chunk: int = 8,
                             relative: bool = False):
    """Device-side batch of low-rank-plus-noise matrices (fp32 arithmetic, stored in ``dtype``);
    ``relative`` as in lowrank_plus_noise."""
    torch = _torch()
    dtype = torch.bfloat16 if dtype is None else dtype
    out = torch.empty(batch, rows, cols, device=device, dtype=dtype)
    r = min(rows, cols)
    s = torch.arange(1, r + 1, device=device, dtype=torch.float32) ** (-power)
    for b0 in range(0, batch, chunk):
        nb = min(chunk, batch - b0)
        gen = _tgen(device, workload_index, seed_offset + b0)
        U = _t_orthonormal(gen, nb, rows, r, device)
        V = _t_orthonormal(gen, nb, cols, r, device)
        G = torch.matmul(U * s, V.transpose(-1, -2).contiguous())
        E = torch.randn(nb, rows, cols, generator=gen, device=device, dtype=torch.float32)
        if relative:
            E *= torch.linalg.vector_norm(s) / torch.linalg.vector_norm(E, dim=(-2, -1), keepdim=True)
        G += noise * E
        if normalize:
            G /= torch.linalg.vector_norm(G, dim=(-2, -1), keepdim=True)
        out[b0:b0 + nb] = G.to(dtype)
    return out


def torch_gaussian_plus_spike(batch: int, rows: int, cols: int, workload_index: int,
                              rank: int = 32, spike_factor: float = 10.0, device="cuda",
                              dtype=None, chunk: int = 16):
    """Device-side batch of N(0,1) matrices plus a rank-``rank`` spike whose singular values are
    ``spike_factor`` x the bulk edge sqrt(rows) + sqrt(cols)."""
    torch = _torch()
    dtype = torch.bfloat16 if dtype is None else dtype
    out = torch.empty(batch, rows, cols, device=device, dtype=dtype)
    sigma = spike_factor * (math.sqrt(rows) + math.sqrt(cols))
    for b0 in range(0, batch, chunk):
        nb = min(chunk, batch - b0)
        gen = _tgen(device, workload_index, b0)
        U = _t_orthonormal(gen, nb, rows, rank, device)
        V = _t_orthonormal(gen, nb, cols, rank, device)
        G = torch.randn(nb, rows, cols, generator=gen, device=device, dtype=torch.float32)
        G += sigma * torch.matmul(U, V.transpose(-1, -2).contiguous())
        out[b0:b0 + nb] = G.to(dtype)
    return out


def torch_loguniform_spectrum(batch: int, rows: int, cols: int, workload_index: int,
                              seed_offset: int = 0, lo: float = 1e-6, hi: float = 1.0,
                              device="cuda", chunk: int = 8):
    """Device-side batch of U diag(s) V^T, s_j = exp(Uniform(ln lo, ln hi)) i.i.d. per matrix,
    random orthonormal U (rows x r) and V (cols x r), r = min(rows, cols); fp32, no noise.
    The caller rounds to the storage dtype."""
    torch = _torch()
    out = torch.empty(batch, rows, cols, device=device, dtype=torch.float32)
    r = min(rows, cols)
    for b0 in range(0, batch, chunk):
        nb = min(chunk, batch - b0)
        gen = _tgen(device, workload_index, seed_offset + b0)
        U = _t_orthonormal(gen, nb, rows, r, device)
        V = _t_orthonormal(gen, nb, cols, r, device)
        u = torch.rand(nb, 1, r, generator=gen, device=device, dtype=torch.float64)
        s = torch.exp(math.log(lo) + (math.log(hi) - math.log(lo)) * u).to(torch.float32)
        out[b0:b0 + nb] = torch.matmul(U * s, V.transpose(-1, -2).contiguous())
    return out


def torch_weights(batch: int, rows: int, cols: int, workload_index: int, std: float = 0.02,
                  device="cuda", dtype=None, seed_offset: int = 500_000):
    """Weights ~ N(0, std^2), stored in ``dtype``."""
    torch = _torch()
    dtype = torch.bfloat16 if dtype is None else dtype
    gen = _tgen(device, workload_index, seed_offset)
    return (std * torch.randn(batch, rows, cols, generator=gen, device=device,
                              dtype=torch.float32)).to(dtype)
