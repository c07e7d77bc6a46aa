"""Mixed-precision Tile-CSC SpMV as a perturbed FP64 operator.

EvoCG models a reduced-precision SpMV as y = (A + E(a)) p (Eq. 2 and Eq. 5):
tile t's entries are read from the value stream its precision code selects
(Sec. 3.3.2), widened exactly, multiplied by the FP64 vector entry and summed
in FP64. The vector is not rounded (a reading: the paper's action names "the
vector tile and its column block", this definition rounds only the matrix).

Two forms are given:

* :func:`spmv_loop` -- serial loops over CSR rows, one product at a time, for
  small inputs.
* :func:`spmv` -- the same sum via SciPy's serial CSR product over the
  per-tile rounded values (a library primitive in place of the inner loop).

The paper's own numerics differ in two ways, offered here as the "P1"
variant (:func:`spmv_p1`, :func:`spmv_p1_loop`):

* the action sets the precision of the vector tile p^(i) as well as of its
  column block (Eq. 9 and Eq. 10), so every product uses the vector entry
  rounded to the tile's precision (then widened exactly);
* the reduced-precision values of a column share one scale factor s_j
  (Sec. 3.3.2, "Intra-Tile CSC Execution"). The factor is not given; the
  reading taken is s_j = 2^e_j with e_j the binary exponent of the column's
  largest |a_ij| (frexp: max = m 2^e, 0.5 <= m < 1), so that the stored FP32
  and BF16 values fl(a_ij / s_j) stay inside those formats' range, and the
  product multiplies the widened value back by s_j exactly in FP64. The FP64
  stream is not scaled.

Test infrastructure only: see the package docstring.
"""

from __future__ import annotations

import numpy as np
import scipy.sparse as sp

from .rounding import stream_values
from .tilecsc import TileCSC


def rounded_csr_values(L: TileCSC, prec_of_tile: np.ndarray) -> np.ndarray:
    """CSR-ordered values where every entry is replaced by its tile's stored value."""
    prec_of_tile = np.asarray(prec_of_tile, dtype=np.uint8)
    if prec_of_tile.size != L.T:
        raise ValueError("map length must equal the number of non-empty tiles")
    prec_nnz = prec_of_tile[L.tile_of_nnz()]
    canon = stream_values(L.val, prec_nnz)
    out = np.empty_like(canon)
    out[L.perm] = canon
    return out


def perturbed_operator(L: TileCSC, indptr, indices, prec_of_tile) -> sp.csr_matrix:
    vals = rounded_csr_values(L, prec_of_tile)
    return sp.csr_matrix((vals, np.asarray(indices), np.asarray(indptr)), shape=(L.n, L.n))


def spmv(L: TileCSC, indptr, indices, prec_of_tile, x) -> np.ndarray:
    """y = (A + E(map)) x with FP64 products and sums, in CSR order."""
    return perturbed_operator(L, indptr, indices, prec_of_tile) @ np.asarray(x, dtype=np.float64)


def spmv_full(n: int, indptr, indices, data, R: int, C: int, prec_of_tile, x, keys=None) -> np.ndarray:
    """Same as :func:`spmv`, for full-size matrices without the whole Tile-CSC object.

    Every CSR entry's tile is found from the sorted tile keys (I * ncb + J, see
    :func:`oracle.tilecsc.tile_numbering`; pass ``keys`` to reuse them), its value is
    replaced by its tile's stored value, and the rounded matrix multiplies x in FP64
    (SciPy's serial CSR product, in CSR order).
    """
    from .tilecsc import tile_numbering, tile_of

    indptr = np.asarray(indptr, dtype=np.int64)
    if keys is None:
        keys, _ = tile_numbering(n, indptr, indices, R, C)
    rows = np.repeat(np.arange(n, dtype=np.int64), np.diff(indptr))
    prec = np.asarray(prec_of_tile, dtype=np.uint8)[tile_of(keys, n, R, C, rows, indices)]
    del rows
    vals = stream_values(np.asarray(data, dtype=np.float64), prec)
    M = sp.csr_matrix((vals, np.asarray(indices), indptr), shape=(n, n))
    return M @ np.asarray(x, dtype=np.float64)


def spmv_loop(L: TileCSC, indptr, indices, prec_of_tile, x) -> np.ndarray:
    """Same as :func:`spmv`, written as plain loops (small inputs only)."""
    vals = rounded_csr_values(L, prec_of_tile)
    y = np.zeros(L.n, dtype=np.float64)
    for i in range(L.n):
        acc = 0.0
        for k in range(int(indptr[i]), int(indptr[i + 1])):
            acc += float(vals[k]) * float(x[int(indices[k])])
        y[i] = acc
    return y


def abs_bound(indptr, indices, data, x) -> np.ndarray:
    """(|A| |x|)_i, the scale of the accuracy bound |y - y_ref|_i <= tol * (|A||x|)_i."""
    A = sp.csr_matrix((np.abs(np.asarray(data)), np.asarray(indices), np.asarray(indptr)))
    return A @ np.abs(np.asarray(x, dtype=np.float64))


def spmv_rows(indptr, indices, data, rows, prec_of_entry, x) -> np.ndarray:
    """y_i for the listed rows only, one plain loop per row.

    ``prec_of_entry(i, cols)`` returns the precision code of row i's entries.
    Used to check full-size products on sampled rows.
    """
    out = np.empty(len(rows), dtype=np.float64)
    for m, i in enumerate(rows):
        s, e = int(indptr[i]), int(indptr[i + 1])
        cols = np.asarray(indices[s:e], dtype=np.int64)
        vals = stream_values(np.asarray(data[s:e], dtype=np.float64), prec_of_entry(int(i), cols))
        acc = 0.0
        for v, c in zip(vals, cols):
            acc += float(v) * float(x[c])
        out[m] = acc
    return out


def column_scale_exponents(n: int, indptr, indices, data) -> np.ndarray:
    """int64[n]: e_j of the per-column scale s_j = 2^e_j (Sec. 3.3.2, reading above).

    e_j is the frexp exponent of max_i |a_ij| over column j, 0 for a column
    without a nonzero value.
    """
    colmax = np.zeros(n, dtype=np.float64)
    np.maximum.at(colmax, np.asarray(indices, dtype=np.int64), np.abs(np.asarray(data, dtype=np.float64)))
    _, e = np.frexp(colmax)
    e = e.astype(np.int64)
    e[colmax == 0.0] = 0
    return e


def p1_stored_values(a: np.ndarray, prec: np.ndarray, col_exp: np.ndarray) -> np.ndarray:
    """Per-entry stored value widened to FP64 with the column scale applied back.

    prec 0: a itself. prec 1 or 2: s_j * fl_prec(a / s_j) with s_j = 2^col_exp
    (both scalings exact in FP64).
    """
    a = np.asarray(a, dtype=np.float64)
    e = np.asarray(col_exp, dtype=np.int64)
    scaled = stream_values(np.ldexp(a, -e), prec)
    return np.where(np.asarray(prec) == 0, a, np.ldexp(scaled, e))


def _csr_entry_precisions(L: TileCSC, prec_of_tile) -> np.ndarray:
    prec_of_tile = np.asarray(prec_of_tile, dtype=np.uint8)
    if prec_of_tile.size != L.T:
        raise ValueError("map length must equal the number of non-empty tiles")
    out = np.empty(L.nnz, dtype=np.uint8)
    out[L.perm] = prec_of_tile[L.tile_of_nnz()]
    return out


def spmv_p1_loop(L: TileCSC, indptr, indices, data, prec_of_tile, x, round_vector=True,
                 col_exp=None) -> np.ndarray:
    """P1 variant as plain loops over CSR rows (small inputs only).

    y_i = sum_j v_ij * x~_j in FP64, CSR order, where v_ij is the stored value
    of entry (i, j) at its tile's precision m (scaled per column when col_exp
    is given) and x~_j is x_j rounded to m when round_vector is set, else x_j.
    """
    indices = np.asarray(indices, dtype=np.int64)
    prec = _csr_entry_precisions(L, prec_of_tile)
    e = np.zeros(L.nnz, dtype=np.int64) if col_exp is None else np.asarray(col_exp, dtype=np.int64)[indices]
    vals = p1_stored_values(np.asarray(data, dtype=np.float64), prec, e)
    x = np.asarray(x, dtype=np.float64)
    y = np.zeros(L.n, dtype=np.float64)
    for i in range(L.n):
        acc = 0.0
        for k in range(int(indptr[i]), int(indptr[i + 1])):
            xj = x[indices[k]]
            if round_vector:
                xj = stream_values(np.array([xj]), np.array([prec[k]]))[0]
            acc += float(vals[k]) * float(xj)
        y[i] = acc
    return y


def spmv_p1(L: TileCSC, indptr, indices, data, prec_of_tile, x, round_vector=True,
            col_exp=None) -> np.ndarray:
    """P1 variant via SciPy: y = sum over m of A_m x~_m, A_m the entries of precision m.

    Sums the three partial products, so its order differs from the loop form;
    the result lies within the same rounding bound.
    """
    indptr = np.asarray(indptr, dtype=np.int64)
    indices = np.asarray(indices, dtype=np.int64)
    prec = _csr_entry_precisions(L, prec_of_tile)
    e = np.zeros(L.nnz, dtype=np.int64) if col_exp is None else np.asarray(col_exp, dtype=np.int64)[indices]
    vals = p1_stored_values(np.asarray(data, dtype=np.float64), prec, e)
    x = np.asarray(x, dtype=np.float64)
    y = np.zeros(L.n, dtype=np.float64)
    for m in (0, 1, 2):
        sel = prec == m
        if not sel.any():
            continue
        Am = sp.csr_matrix((np.where(sel, vals, 0.0), indices, indptr), shape=(L.n, L.n))
        xm = stream_values(x, np.full(x.size, m, dtype=np.uint8)) if round_vector else x
        y += Am @ xm
    return y
