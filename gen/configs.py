"""The five workloads, their seeds and their precision-map specifications.

Precision codes follow the EvoCG action encoding (paper Sec. 3.2.2, Eq. 9):
0 = FP64, 1 = FP32, 2 = BF16.

Seeds: x* uses ``default_rng(0)``; matrix randomness (coefficients,
structure, values) uses ``default_rng(1)``; per-tile scores use
``default_rng(2)``. Right-hand sides are b = A x* with the exact FP64
matrix, and x0 = 0 everywhere.

``scale="full"`` gives the sizes the benchmark and the full-size parity
tests use. ``scale="small"`` gives versions the CPU oracle solves in
seconds; they keep the structure and value distribution, span many tiles
and have a ragged last row block.
"""

from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

from .matrices import (
    CSR,
    aniso2d_q1,
    diffusion3d_27pt,
    laplace2d_5pt,
    laplace3d_7pt,
    random_spd_powerlaw,
)

FP64, FP32, BF16 = 0, 1, 2


@dataclass
class Workload:
    name: str
    description: str
    A: CSR
    R: int
    C: int
    xstar: np.ndarray
    b: np.ndarray
    tol: float
    maxit: int
    map_spec: dict
    jacobi: bool = False
    meta: dict = field(default_factory=dict)

    @property
    def n(self) -> int:
        return self.A.n

    def input_hash(self) -> str:
        """Digest of every input array and parameter (for caching oracle results)."""
        h = hashlib.sha256()
        for arr in (self.A.indptr, self.A.indices, self.A.data, self.b):
            h.update(np.ascontiguousarray(arr).tobytes())
        h.update(repr((self.R, self.C, self.tol, self.maxit, sorted(self.map_spec.items()),
                       self.jacobi)).encode())
        return h.hexdigest()[:16]


CONFIGS = {
    1: dict(full=dict(m=64), small=dict(m=64)),
    2: dict(full=dict(m=128), small=dict(m=21)),
    3: dict(full=dict(m=100), small=dict(m=21)),
    4: dict(full=dict(n=4_000_000), small=dict(n=20_011)),
    5: dict(full=dict(m=4096), small=dict(m=100)),
}


def tile_scores(T: int, seed: int = 2) -> np.ndarray:
    """Per-tile scores s_t ~ U[0, 1), one per non-empty tile in canonical tile order."""
    return np.random.default_rng(seed).random(int(T))


def static_map(scores: np.ndarray, frac_bf16: float = 0.2, frac_fp32: float = 0.3) -> np.ndarray:
    """A seeded static per-tile map: BF16 if s < f_bf16, FP32 if s < f_bf16 + f_fp32, else FP64."""
    m = np.full(scores.shape, FP64, dtype=np.uint8)
    m[scores < frac_bf16 + frac_fp32] = FP32
    m[scores < frac_bf16] = BF16
    return m


def _rhs(A: CSR):
    xstar = np.random.default_rng(0).uniform(-1.0, 1.0, A.n)
    return xstar, A.matvec(xstar)


def make_workload(cfg: int, scale: str = "small") -> Workload:
    p = CONFIGS[cfg][scale]
    if cfg == 1:
        A = laplace2d_5pt(p["m"])
        desc = f"2D 5-point Laplacian {p['m']}^2, 16x16 tiles, all-FP64 map"
        R = C = 16
        tol, maxit = 1e-10, 500
        spec = dict(kind="fp64")
        jac = False
    elif cfg == 2:
        A = laplace3d_7pt(p["m"])
        desc = f"3D 7-point Laplacian {p['m']}^3, 16x16 tiles, static 50/30/20 FP64/FP32/BF16 map"
        R = C = 16
        tol, maxit = 1e-8, 10_000
        spec = dict(kind="static", frac_bf16=0.2, frac_fp32=0.3, seed=2)
        jac = False
    elif cfg == 3:
        A = diffusion3d_27pt(p["m"], seed=1)
        desc = (f"3D 27-point variable-coefficient diffusion {p['m']}^3, 16x16 tiles, "
                "magnitude-rule map")
        R = C = 16
        tol, maxit = 1e-8, 10_000
        spec = dict(kind="magnitude", t_bf16=1e-4, t_fp32=1e-2)
        jac = False
    elif cfg == 4:
        A = random_spd_powerlaw(p["n"], seed=1)
        desc = (f"random SPD n={p['n']}, band 8 + power-law rows, 16x16 tiles, Jacobi-PCG, "
                "residual-ratchet map BF16->FP32->FP64")
        R = C = 16
        tol, maxit = 1e-10, 10_000
        spec = dict(kind="ratchet", thresholds=(1e-3, 1e-6), prec=(BF16, FP32, FP64))
        jac = True
    elif cfg == 5:
        A = aniso2d_q1(p["m"])
        desc = (f"2D 9-point Q1 anisotropic (1, 1e-3) {p['m']}^2, 32x32 tiles, per-tile "
                "re-selection every 10 iterations")
        R = C = 32
        tol, maxit = 1e-9, 5000
        spec = dict(kind="tile_rule", period=10, hi=1e-3, lo=1e-6, seed=2)
        jac = False
    else:
        raise ValueError(f"unknown config {cfg}")
    xstar, b = _rhs(A)
    return Workload(name=f"cfg{cfg}-{scale}", description=desc, A=A, R=R, C=C, xstar=xstar,
                    b=b, tol=tol, maxit=maxit, map_spec=spec, jacobi=jac)
