"""Textbook FP64 CG and Jacobi-PCG around the perturbed SpMV.

Follows the CG recurrence of the EvoCG paper (Sec. 2.1, Eq. 1, Fig. 1, and
the solver lines of Algorithm 1): one SpMV, two dot products and three AXPYs
per iteration,

    alpha = (r.r) / (p.q),  x += alpha p,  r_new = r - alpha q,
    beta = (r_new.r_new) / (r.r),  p = r_new + beta p,

with q = (A + E(a_k)) p the mixed-precision product (Eq. 5). The stopping
rule is the recurrence residual ||r_k|| / ||r_0|| <= tol or k = max_iter,
checked at the top of every iteration (Algorithm 1's loop header; Sec. 4.1
"Unified solver configuration"). Jacobi-PCG (Sec. 4.6) keeps the precision
control on q = A p only; z = M^-1 r with M = diag(A), every scalar in FP64,
and the stop still uses the unpreconditioned residual.

Conventions taken where the paper is silent:

* x0 = 0 unless given; r0 = b - A x0 with the exact FP64 matrix.
* K counts completed iterations; ``hist`` holds rho_0 .. rho_K with rho_0 = 1.
* p.q <= 0 or a non-finite alpha/beta stops with status "breakdown".
* ||r0|| = 0 returns x0 with K = 0 and hist = [0].
* The map for iteration k is chosen from (k, rho_k) -- or, for the per-segment
  max|p| rule, from the direction p_k -- by a schedule.

Test infrastructure only: see the package docstring.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import scipy.sparse as sp

from . import maps as _maps
from .rounding import stream_values, to_bf16_value, to_fp32
from .spmv import column_scale_exponents, p1_stored_values
from .tilecsc import TileCSC


class StaticSchedule:
    def __init__(self, prec_map):
        self.map = np.asarray(prec_map, dtype=np.uint8)

    def map_for(self, k, rho, T, p=None):
        return self.map if k == 0 else None


class RatchetSchedule:
    def __init__(self, thresholds, prec):
        self.r = _maps.Ratchet(thresholds, prec)
        self.current = None

    def map_for(self, k, rho, T, p=None):
        code = self.r.step(rho)
        if code != self.current:
            self.current = code
            return np.full(T, code, dtype=np.uint8)
        return None


class TileRuleSchedule:
    def __init__(self, scores, period, hi, lo):
        self.scores = np.asarray(scores, dtype=np.float64)
        self.period = int(period)
        self.hi, self.lo = float(hi), float(lo)

    def map_for(self, k, rho, T, p=None):
        if k % self.period == 0:
            return _maps.tile_rule(self.scores, rho, self.hi, self.lo)
        return None


class PMagSchedule:
    """The per-segment max|p| rule (Sec. 4.7), applied to the direction p_k that the
    iteration's SpMV multiplies, at every iteration whose index is a multiple of
    ``period`` and reused in between (Sec. 3.4 "Interval Reuse Scheduling").
    ``column_codes``, when a list, receives every evaluation's per-column-block
    codes."""

    def __init__(self, C, tile_col_idx, lo, hi, period=1, column_codes=None):
        self.C = int(C)
        self.tcol = np.asarray(tile_col_idx)
        self.lo, self.hi = float(lo), float(hi)
        self.period = int(period)
        self.column_codes = column_codes

    def map_for(self, k, rho, T, p=None):
        if k % self.period != 0:
            return None
        if self.column_codes is not None:
            self.column_codes.append(_maps.pmag_column_codes(p, self.C, self.lo, self.hi))
        return _maps.pmag_rule(p, self.C, self.tcol, self.lo, self.hi)


@dataclass
class Result:
    x: np.ndarray
    K: int
    hist: list
    status: str
    windows: list = field(default_factory=list)  # (k, counts[3], map) at every map change
    true_residual: float = float("nan")


def _row_order(indptr, reverse):
    """Storage positions of the CSR entries in the order each row is summed: as stored, or
    every row reversed. Both are plain sums of the same terms; only the rounding differs."""
    indptr = np.asarray(indptr, dtype=np.int64)
    nnz = int(indptr[-1])
    if not reverse:
        return np.arange(nnz, dtype=np.int64)
    row = np.repeat(np.arange(indptr.size - 1, dtype=np.int64), np.diff(indptr))
    pos = np.arange(nnz, dtype=np.int64)
    return (indptr[row] + indptr[row + 1] - 1 - pos).astype(np.int64)


class PerturbedOperator:
    """Holds the three value streams in CSR order and forms (A + E(map)) on demand.

    reverse_rows sums every row of the product in reverse storage order (the same terms in
    another order), for telling rounding-order effects from errors."""

    def __init__(self, L: TileCSC, indptr, indices, data, reverse_rows=False):
        self.n = L.n
        self.T = L.T
        tile_canon = L.tile_of_nnz()
        tile_of_csr = np.empty_like(tile_canon)
        tile_of_csr[L.perm] = tile_canon
        order = _row_order(indptr, reverse_rows)
        self.tile_of_csr = tile_of_csr[order]
        a = np.asarray(data, dtype=np.float64)[order]
        self.streams = (a, to_fp32(a).astype(np.float64), to_bf16_value(a))
        self.M = sp.csr_matrix((a.copy(), np.asarray(indices)[order], np.asarray(indptr)),
                               shape=(L.n, L.n))

    def set_map(self, prec_map):
        prec_nnz = np.asarray(prec_map, dtype=np.uint8)[self.tile_of_csr]
        self.M.data = np.choose(prec_nnz, self.streams)

    def __matmul__(self, p):
        return self.M @ p


class P1Operator:
    """The paper's own product: the vector entry rounded with its tile (Eq. 9/10).

    Entry (i, j) of a tile at precision m contributes v_ij * p~_j in FP64,
    where v_ij is the stored value (scaled per column when column_scale is
    set, Sec. 3.3.2) and p~_j is p_j rounded to m when round_vector is set.
    The product is taken as sum over m of A_m p~^(m), A_m holding the entries
    at precision m.
    """

    def __init__(self, L: TileCSC, indptr, indices, data, round_vector=True, column_scale=False,
                 reverse_rows=False):
        self.n = L.n
        tile_canon = L.tile_of_nnz()
        tile_of_csr = np.empty_like(tile_canon)
        tile_of_csr[L.perm] = tile_canon
        order = _row_order(indptr, reverse_rows)
        self.tile_of_csr = tile_of_csr[order]
        self.indptr = np.asarray(indptr)
        self.indices = np.asarray(indices)[order]
        a = np.asarray(data, dtype=np.float64)
        e = (column_scale_exponents(L.n, indptr, indices, a)[self.indices] if column_scale
             else np.zeros(a.size, dtype=np.int64))
        a = a[order]
        self.streams = tuple(p1_stored_values(a, np.full(a.size, m, np.uint8), e) for m in (0, 1, 2))
        self.round_vector = round_vector
        self.parts = []

    def set_map(self, prec_map):
        prec_nnz = np.asarray(prec_map, dtype=np.uint8)[self.tile_of_csr]
        self.parts = []
        for m in (0, 1, 2):
            sel = prec_nnz == m
            if sel.any():
                Am = sp.csr_matrix((np.where(sel, self.streams[m], 0.0), self.indices, self.indptr),
                                   shape=(self.n, self.n))
                self.parts.append((m, Am))

    def __matmul__(self, p):
        y = np.zeros(self.n)
        for m, Am in self.parts:
            pm = stream_values(p, np.full(p.size, m, np.uint8)) if self.round_vector else p
            y += Am @ pm
        return y


def solve(L: TileCSC, indptr, indices, data, b, schedule, tol, maxit, x0=None,
          jacobi=False, trace=None, keep_maps=True, round_vector=False,
          column_scale=False, reverse_rows=False) -> Result:
    """CG (or Jacobi-PCG) with the mixed-precision product.

    round_vector / column_scale select the paper's own product (P1Operator);
    r0 = b - A x0 always uses the exact FP64 matrix. reverse_rows sums the product's rows in
    reverse storage order: a second correct rounding of the same iteration, whose distance
    from the first shows how far rounding order alone moves a run.
    """
    n = L.n
    A = sp.csr_matrix((np.asarray(data, dtype=np.float64), np.asarray(indices),
                       np.asarray(indptr)), shape=(n, n))
    if round_vector or column_scale:
        op = P1Operator(L, indptr, indices, data, round_vector, column_scale, reverse_rows)
    else:
        op = PerturbedOperator(L, indptr, indices, data, reverse_rows)
    b = np.asarray(b, dtype=np.float64)
    x = np.zeros(n) if x0 is None else np.array(x0, dtype=np.float64)
    r = b - A @ x
    if jacobi:
        dinv = 1.0 / A.diagonal()
        z = dinv * r
    else:
        z = r
    p = z.copy()
    rr = float(np.dot(r, r))
    rz = float(np.dot(r, z))
    norm0 = math.sqrt(rr)
    windows = []
    if norm0 == 0.0:
        res = Result(x=x, K=0, hist=[0.0], status="converged", windows=windows)
        res.true_residual = _true_residual(A, x, b)
        return res
    hist = [1.0]
    k = 0
    status = "maxit"
    while True:
        rho = hist[-1]
        if rho <= tol:
            status = "converged"
            break
        if k == maxit:
            status = "maxit"
            break
        new_map = schedule.map_for(k, rho, L.T, p)
        if new_map is not None:
            op.set_map(new_map)
            counts = np.bincount(new_map, minlength=3)[:3].tolist()
            windows.append((k, counts, new_map.copy() if keep_maps else None))
        q = op @ p
        pq = float(np.dot(p, q))
        if not (pq > 0.0) or not math.isfinite(pq):
            status = "breakdown"
            break
        alpha = rz / pq
        if not math.isfinite(alpha):
            # p.q > 0 but so small that r.z / p.q overflows: a breakdown found
            # before the update, so the iterate and K stay as they are.
            status = "breakdown"
            break
        if trace is not None:
            trace(k, x, r, p, q, alpha)
        x += alpha * p
        r -= alpha * q
        rr_new = float(np.dot(r, r))
        if jacobi:
            z = dinv * r
            rz_new = float(np.dot(r, z))
        else:
            z = r
            rz_new = rr_new
        beta = rz_new / rz
        if not math.isfinite(beta):
            status = "breakdown"
            k += 1
            hist.append(math.sqrt(rr_new) / norm0)
            break
        p = z + beta * p
        rz = rz_new
        k += 1
        hist.append(math.sqrt(rr_new) / norm0)
    res = Result(x=x, K=k, hist=hist, status=status, windows=windows)
    res.true_residual = _true_residual(A, x, b)
    return res


def _true_residual(A, x, b):
    nb = float(np.linalg.norm(b))
    r = b - A @ x
    return float(np.linalg.norm(r)) / nb if nb > 0 else float(np.linalg.norm(r))


def schedule_for(spec: dict, L: TileCSC, scores=None, static=None):
    """Build the schedule that a workload's map specification describes."""
    kind = spec["kind"]
    if kind == "fp64":
        return StaticSchedule(np.zeros(L.T, dtype=np.uint8))
    if kind == "static":
        return StaticSchedule(static)
    if kind == "magnitude":
        return StaticSchedule(_maps.magnitude_rule(L, spec["t_bf16"], spec["t_fp32"]))
    if kind == "ratchet":
        return RatchetSchedule(spec["thresholds"], spec["prec"])
    if kind == "tile_rule":
        return TileRuleSchedule(scores, spec["period"], spec["hi"], spec["lo"])
    if kind == "pmag":
        return PMagSchedule(L.C, L.tile_col_idx, spec["lo"], spec["hi"], spec.get("period", 1))
    raise ValueError(kind)
