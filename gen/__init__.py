"""Seeded synthetic inputs shared by the oracle, the tests and the benchmark.

This package draws random numbers and assembles the five SPD test matrices
in CSR form. It holds none of the solver's arithmetic: no tiling, no
rounding to FP32/BF16, no SpMV of the method and no CG. Both the CPU oracle
and the HIP path consume exactly these arrays.

The five workloads stand in for the SuiteSparse SPD collection that the
EvoCG paper evaluates on ("EvoCG: Self-Evolving Precision Control for
Faster Conjugate Gradient", Sec. 4.1 "Datasets"), which is not available
here. Each builder documents its construction.
"""

from .matrices import (  # noqa: F401
    CSR,
    laplace2d_5pt,
    laplace3d_7pt,
    diffusion3d_27pt,
    random_spd_powerlaw,
    aniso2d_q1,
)
from .configs import CONFIGS, Workload, make_workload, tile_scores, static_map  # noqa: F401
