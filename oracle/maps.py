"""Precision-map rules of the five workloads (codes 0 = FP64, 1 = FP32, 2 = BF16).

The EvoCG paper selects tile precisions with a learned policy (Sec. 3.2),
which is out of scope here; the workloads use rules instead. The paper fixes
the action encoding (Eq. 9: a in {0, 1, 2} for {FP64, FP32, BF16}) and the
idea of re-selecting a map at the start of a reuse window and keeping it for
the window (Sec. 3.4, "Interval Reuse Scheduling"). Every rule below is a
reading of a workload description and is applied per tile.

Test infrastructure only: see the package docstring.
"""

from __future__ import annotations

import numpy as np

from .tilecsc import TileCSC

FP64, FP32, BF16 = 0, 1, 2


def magnitude_rule(L: TileCSC, t_bf16: float = 1e-4, t_fp32: float = 1e-2) -> np.ndarray:
    """Map from ratio_t = max_{(i,j) in t} |a_ij| / max_i |a_ii| (global diagonal max).

    BF16 if ratio_t < t_bf16, FP32 if ratio_t < t_fp32, else FP64 (strict
    comparisons, FP64 division).
    """
    tile = L.tile_of_nnz()
    rb = L.tile_row_block()[tile]
    rows = rb * L.R + L.row_idx.astype(np.int64)
    cols = L.tile_col_idx.astype(np.int64)[tile] * L.C + L.local_col()
    absval = np.abs(L.val)
    diag = absval[rows == cols]
    dmax = float(diag.max()) if diag.size else 0.0
    tmax = np.zeros(L.T, dtype=np.float64)
    np.maximum.at(tmax, tile, absval)
    ratio = tmax / dmax
    out = np.full(L.T, FP64, dtype=np.uint8)
    out[ratio < t_fp32] = FP32
    out[ratio < t_bf16] = BF16
    return out


class Ratchet:
    """One-way residual schedule: the map for iteration k depends on rho_k = ||r_k|| / ||r_0||.

    ``prec[0]`` applies until rho <= thresholds[0] has been seen, ``prec[1]``
    until rho <= thresholds[1] has been seen, and so on; a stage once reached
    is never left. The map is uniform over all tiles.
    """

    def __init__(self, thresholds, prec):
        self.thresholds = [float(t) for t in thresholds]
        self.prec = [int(p) for p in prec]
        if len(self.prec) != len(self.thresholds) + 1:
            raise ValueError("need one more precision than thresholds")
        self.stage = 0

    def step(self, rho: float) -> int:
        while self.stage < len(self.thresholds) and rho <= self.thresholds[self.stage]:
            self.stage += 1
        return self.prec[self.stage]


def pmag_rule(p: np.ndarray, C: int, tile_col_idx: np.ndarray, lo: float, hi: float) -> np.ndarray:
    """Residual-threshold rule on the direction vector (Sec. 4.7 "Why Learned Precision Control?").

    Tile t reads its column block J = tile_col_idx[t], i.e. the segment
    p[J*C : (J+1)*C] of the vector it multiplies (the last segment may be
    shorter). With m_J = max |p_j| over that segment: BF16 if m_J < lo, FP32 if
    lo <= m_J < hi, FP64 otherwise. The paper's setting is lo = eps/10, hi = eps
    for the solver tolerance eps.
    """
    p = np.abs(np.asarray(p, dtype=np.float64))
    n = p.size
    ncb = -(-n // C)
    pad = np.zeros(ncb * C)
    pad[:n] = p
    m = pad.reshape(ncb, C).max(axis=1)
    mt = m[np.asarray(tile_col_idx, dtype=np.int64)]
    out = np.full(mt.shape, FP64, dtype=np.uint8)
    out[mt < hi] = FP32
    out[mt < lo] = BF16
    return out


def pmag_column_codes(p: np.ndarray, C: int, lo: float, hi: float) -> np.ndarray:
    """The max|p| rule's code of every column block (uint8[ceil(n/C)]); see pmag_rule."""
    p = np.abs(np.asarray(p, dtype=np.float64))
    ncb = -(-p.size // C)
    pad = np.zeros(ncb * C)
    pad[:p.size] = p
    m = pad.reshape(ncb, C).max(axis=1)
    out = np.full(ncb, FP64, dtype=np.uint8)
    out[m < hi] = FP32
    out[m < lo] = BF16
    return out


def delayed_upward_fraction(codes: np.ndarray, interval: int) -> float:
    """Interval reuse (Sec. 3.4 "Interval Reuse Scheduling") applied to a per-iteration record.

    ``codes[k, J]`` is column block J's code at iteration k of a per-iteration
    run (0 = FP64 > 1 = FP32 > 2 = BF16 in precision). An upward transition is
    a (k, J) with k >= 1 and codes[k, J] < codes[k-1, J]. Reusing decisions over
    windows of ``interval`` iterations gives iteration k the decision of its
    window start s = (k // interval) * interval; the transition is delayed when
    that decision is of lower precision than the one at k (codes[s, J] >
    codes[k, J]). Returns delayed / upward, or 0 when there is no upward
    transition.
    """
    codes = np.asarray(codes)
    K = codes.shape[0]
    if K < 2:
        return 0.0
    up = codes[1:] < codes[:-1]
    ks = np.arange(1, K)
    start = codes[(ks // int(interval)) * int(interval)]
    delayed = up & (start > codes[1:])
    n_up = int(up.sum())
    return float(delayed.sum()) / n_up if n_up else 0.0


def select_reuse_interval(codes: np.ndarray, max_fraction: float = 0.1) -> tuple:
    """K* (Sec. 3.4): the largest candidate interval 1, 2, 4, ... (below the number
    of recorded iterations) whose delayed-upward fraction is below ``max_fraction``.

    Returns (K*, [(interval, fraction), ...]) over the candidates tried.
    """
    K = np.asarray(codes).shape[0]
    best, table, interval = 1, [], 1
    while interval < max(K, 2):
        f = delayed_upward_fraction(codes, interval)
        table.append((interval, f))
        if f < max_fraction:
            best = interval
        interval *= 2
    return best, table


def tile_rule(scores: np.ndarray, rho: float, hi: float = 1e-3, lo: float = 1e-6) -> np.ndarray:
    """Per-tile re-selection: v_t = s_t * rho; BF16 if v_t > hi, FP32 if v_t > lo, else FP64."""
    v = np.asarray(scores, dtype=np.float64) * float(rho)
    out = np.full(v.shape, FP64, dtype=np.uint8)
    out[v > lo] = FP32
    out[v > hi] = BF16
    return out
