"""Row-block height tuning (EvoCG, Sec. 3.3.3 "Cross-Level Balance Tuning").

The paper fixes the tile width C and tunes the row-block height R over the
powers of two 32, 64, ..., 16384 so that the row blocks hold similar numbers
of non-empty tiles. It names neither the measure of evenness nor what keeps
the search from the trivial answer (a handful of huge row blocks is
perfectly even and leaves the device idle). The reading taken here:

* evenness is the coefficient of variation (population standard deviation
  over mean) of the non-empty tile counts of all ceil(n / R) row blocks,
  computed from exact integer sums (see :func:`balance`);
* a candidate must leave at least ``min_row_blocks`` row blocks, and it must
  not exceed ``max_R`` (the largest height the kernel supports);
* the tuned R is the admissible candidate with the smallest coefficient of
  variation, ties going to the smaller R; with no admissible candidate it is
  the smallest candidate.

Test infrastructure only: see the package docstring.
"""

from __future__ import annotations

import math

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
    """(coefficient of variation, max / mean) of the row blocks' tile counts (0, 0 when all are empty).

    With m row blocks, S1 = sum c and S2 = sum c^2 (exact integers), the
    population standard deviation over the mean is sqrt(m S2 - S1^2) / S1 and
    max / mean is m max(c) / S1. Each is evaluated from the exact integers with
    one rounding to FP64 per operand and IEEE sqrt and division, so the value,
    and with it the choice between near-equal candidates, does not depend on a
    summation order.
    """
    c = [int(v) for v in np.asarray(counts).ravel()]
    m, s1 = len(c), sum(c)
    if s1 == 0:
        return 0.0, 0.0
    s2 = sum(v * v for v in c)
    return math.sqrt(float(m * s2 - s1 * s1)) / float(s1), float(m * max(c)) / float(s1)


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
