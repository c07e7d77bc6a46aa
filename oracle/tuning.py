"""Row-block height tuning (EvoCG, Sec. 3.3.3 "Cross-Level Balance Tuning").

The paper fixes the tile width C and tunes the row-block height R over the
powers of two 32, 64, ..., 16384 so that the row blocks hold similar numbers
of non-empty tiles. It names neither the measure of evenness nor what keeps
the search from the trivial answer (a handful of huge row blocks is
perfectly even and leaves the device idle). The reading taken here:

* evenness is the coefficient of variation (population standard deviation
  over mean) of the non-empty tile counts of all ceil(n / R) row blocks;
  candidates are compared by its exact square (rational arithmetic, see
  :func:`cv_squared`), so that two candidates a floating-point evaluation
  cannot tell apart are still ordered correctly;
* a candidate must leave at least ``min_row_blocks`` row blocks, and it must
  not exceed ``max_R`` (by default the largest candidate, so every candidate
  height the paper lists is admissible);
* the tuned R is the admissible candidate with the smallest coefficient of
  variation, ties going to the smaller R; with no admissible candidate it is
  the smallest candidate.

Test infrastructure only: see the package docstring.
"""

from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

CANDIDATES = tuple(32 << i for i in range(10))  # 32, 64, ..., 16384


def row_block_tile_counts(n: int, indptr, indices, R: int, C: int) -> np.ndarray:
    """int64[ceil(n/R)]: number of non-empty R x C tiles in every row block."""
    indptr = np.asarray(indptr, dtype=np.int64)
    rows = np.repeat(np.arange(n, dtype=np.int64), np.diff(indptr))
    ncb = -(-n // C)
    keys = np.unique((rows // R) * ncb + np.asarray(indices, dtype=np.int64) // C)
    return np.bincount(keys // ncb, minlength=-(-n // R)).astype(np.int64)


def cv_squared(counts) -> Fraction:
    """Exact square of the coefficient of variation of ``counts`` (0 when all are zero).

    Written from the definition: mean = sum(c) / m, population variance =
    sum((c - mean)^2) / m, and cv^2 = variance / mean^2, all in rational
    arithmetic. Equal counts are grouped first (a library primitive), which
    changes nothing in the exact sum.
    """
    values, mult = np.unique(np.asarray(counts, dtype=np.int64).ravel(), return_counts=True)
    m = int(mult.sum())
    total = sum(int(v) * int(k) for v, k in zip(values, mult))
    if m == 0 or total == 0:
        return Fraction(0)
    mean = Fraction(total, m)
    var = sum(int(k) * (int(v) - mean) ** 2 for v, k in zip(values, mult)) / m
    return var / (mean * mean)


def balance(counts: np.ndarray):
    """(coefficient of variation, max / mean) of the row blocks' tile counts (0, 0 when all are empty).

    Both are the exact values rounded to FP64 (the square root of the exact
    cv^2 rounded once, then one IEEE square root); the selection compares the
    exact cv^2 itself.
    """
    c = np.asarray(counts, dtype=np.int64).ravel()
    total = int(c.sum())
    if total == 0:
        return 0.0, 0.0
    return math.sqrt(float(cv_squared(c))), float(Fraction(len(c) * int(c.max()), total))


def select_height(candidates, max_R: int = 16384, min_row_blocks: int = 1024) -> int:
    """The tuned R from (R, counts) pairs in candidate order (Sec. 3.3.3 reading above).

    Admissible: R <= max_R and at least ``min_row_blocks`` row blocks. The
    smallest exact cv^2 wins; on equal cv^2 the earlier (smaller) R stays;
    with no admissible candidate, the first candidate's R.
    """
    best = None
    for R, counts in candidates:
        if R <= max_R and len(counts) >= min_row_blocks:
            v = cv_squared(counts)
            if best is None or v < best[1]:
                best = (R, v)
    return best[0] if best is not None else candidates[0][0]


def tune_row_height(n: int, indptr, indices, C: int, max_R: int = 16384, min_row_blocks: int = 1024,
                    candidates=CANDIDATES):
    """Tuned R and one table row per candidate: (R, row blocks, tiles, cv, max/mean, admissible)."""
    table, pairs = [], []
    for R in candidates:
        counts = row_block_tile_counts(n, indptr, indices, R, C)
        cv, mx = balance(counts)
        ok = R <= max_R and counts.size >= min_row_blocks
        table.append((R, int(counts.size), int(counts.sum()), cv, mx, ok))
        pairs.append((R, counts))
    return select_height(pairs, max_R, min_row_blocks), table
