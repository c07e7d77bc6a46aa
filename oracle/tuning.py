"""Row-block height tuning (EvoCG, Sec. 3.3.3 "Cross-Level Balance Tuning").

The paper fixes the tile width C and tunes the row-block height R over the
powers of two 32, 64, ..., 16384 so that the row blocks hold similar numbers
of non-empty tiles. It names neither the measure of evenness nor what keeps
the search from the trivial answer (a handful of huge row blocks is
perfectly even and leaves the device idle). The reading taken here:

* evenness is the coefficient of variation (population standard deviation
  over mean) of the non-empty tile counts of all ceil(n / R) row blocks;
* a candidate must leave at least ``min_row_blocks`` row blocks, and it must
  not exceed ``max_R`` (the largest height the kernel supports);
* the tuned R is the admissible candidate with the smallest coefficient of
  variation, ties going to the smaller R; with no admissible candidate it is
  the smallest candidate.

Test infrastructure only: see the package docstring.
"""

from __future__ import annotations

import numpy as np

CANDIDATES = tuple(32 << i for i in range(10))  # 32, 64, ..., 16384


def row_block_tile_counts(n: int, indptr, indices, R: int, C: int) -> np.ndarray:
    """int64[ceil(n/R)]: number of non-empty R x C tiles in every row block."""
    indptr = np.asarray(indptr, dtype=np.int64)
    rows = np.repeat(np.arange(n, dtype=np.int64), np.diff(indptr))
    ncb = -(-n // C)
    keys = np.unique((rows // R) * ncb + np.asarray(indices, dtype=np.int64) // C)
    return np.bincount(keys // ncb, minlength=-(-n // R)).astype(np.int64)


def balance(counts: np.ndarray):
    """(coefficient of variation, max / mean) of a row block's tile counts (0, 0 when all are empty)."""
    counts = np.asarray(counts, dtype=np.float64)
    mean = counts.mean()
    if mean == 0.0:
        return 0.0, 0.0
    return float(counts.std() / mean), float(counts.max() / mean)


def tune_row_height(n: int, indptr, indices, C: int, max_R: int = 256, min_row_blocks: int = 1024,
                    candidates=CANDIDATES):
    """Tuned R and one table row per candidate: (R, row blocks, tiles, cv, max/mean, admissible)."""
    table = []
    best = None
    for R in candidates:
        counts = row_block_tile_counts(n, indptr, indices, R, C)
        cv, mx = balance(counts)
        ok = R <= max_R and counts.size >= min_row_blocks
        table.append((R, int(counts.size), int(counts.sum()), cv, mx, ok))
        if ok and (best is None or cv < best[1]):
            best = (R, cv)
    return (best[0] if best is not None else candidates[0]), table
