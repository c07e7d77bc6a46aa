"""CPU oracle for mixed-precision Tile-CSC Conjugate Gradient.

TEST INFRASTRUCTURE ONLY. Nothing in the library or its Python binding may
import this package; only the tests, the smoke check and the benchmark's
CPU-baseline leg do. It shares no code with the HIP path.

It is a plain, serial, FP64 restatement of what the EvoCG paper ("EvoCG:
Self-Evolving Precision Control for Faster Conjugate Gradient") computes:

* ``tilecsc``   -- the canonical Tile-CSC layout (Sec. 3.3, Fig. 4(a)/(b)).
* ``rounding``  -- the three value streams FP64 / FP32 / BF16 (Sec. 3.3.2).
* ``spmv``      -- the perturbed operator (A + E(a)) p of Eq. (2)/(5), with
  every tile's values rounded to its mapped precision and every product and
  sum in FP64; and the paper's own variant ("P1"), which also rounds the
  vector entry to the tile's precision (Eq. 9/10) and scales reduced-precision
  values per column (Sec. 3.3.2).
* ``maps``      -- the precision-map rules used by the workloads.
* ``cg``        -- textbook CG (Fig. 1, Algorithm 1's solver lines) and
  Jacobi-PCG (Sec. 4.6), with the stopping rule of Sec. 4.1.
* ``tuning``    -- the row-block height search of Sec. 3.3.3 (non-empty tile
  counts per row block, their evenness, the tuned R).

Pins (tests marked ``not gpu``) tie every function to something other than
itself: brute force on tiny inputs, library routines on special cases,
closed forms and CG invariants. No function here is "parity unpinned".
"""

from . import rounding, tilecsc, spmv, maps, cg, tuning  # noqa: F401
