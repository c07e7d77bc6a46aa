"""Mixed-precision Tile-CSC SpMV as a perturbed FP64 operator.

EvoCG models a reduced-precision SpMV as y = (A + E(a)) p (Eq. 2 and Eq. 5):
tile t's entries are read from the value stream its precision code selects
(Sec. 3.3.2), widened exactly, multiplied by the FP64 vector entry and summed
in FP64. The vector is not rounded (a reading: the paper's action names "the
vector tile and its column block", this build rounds only the matrix).

Two forms are given:

* :func:`spmv_loop` -- serial loops over CSR rows, one product at a time, for
  small inputs.
* :func:`spmv` -- the same sum via SciPy's serial CSR product over the
  per-tile rounded values (a library primitive in place of the inner loop).

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
