"""Canonical Tile-CSC layout, restated from the EvoCG paper, Sec. 3.3 and Fig. 4.

Definition used here (Fig. 4(a) inter-tile CSR, Fig. 4(b) intra-tile CSC):

* The matrix is cut into R x C tiles; tile (I, J) covers rows [I*R, (I+1)*R)
  and columns [J*C, (J+1)*C).
* Non-empty tiles are listed row block by row block, and by ascending column
  block inside a row block. ``tile_row_ptr[I]..tile_row_ptr[I+1]`` delimits
  row block I's tiles; ``tile_col_idx[t]`` is tile t's column block.
* Inside a tile the nonzeros are stored column by column (CSC):
  ``col_ptr[t, c]`` (relative to the tile's first nonzero) starts local
  column c (derived on demand from the per-nonzero local column), ``row_idx`` holds the row offset from the row block's first row,
  ascending inside a column. ``tile_nnz_ptr`` is the prefix sum of the tiles'
  nonzero counts, so tile t owns positions
  ``tile_nnz_ptr[t]..tile_nnz_ptr[t+1]`` of every per-nonzero array.
* ``perm[k]`` is the CSR position of canonical nonzero k, so the canonical
  FP64 values are ``data[perm]``.

The paper pads columns to an even count with sentinel rows (Sec. 3.3.2);
that is storage detail and not part of the canonical layout here. The padded
view of Fig. 4(b) is available per tile as :func:`padded_columns` and for the
whole matrix as :func:`padded_layout`.

Test infrastructure only: see the package docstring.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass
class TileCSC:
    n: int
    R: int
    C: int
    tile_row_ptr: np.ndarray  # int64[nRB+1]
    tile_col_idx: np.ndarray  # int32[T]
    tile_nnz_ptr: np.ndarray  # int64[T+1]
    row_idx: np.ndarray       # uint16[nnz]  (R <= 16384)
    col_local: np.ndarray     # uint8[nnz]   local column of every nonzero (C <= 256)
    perm: np.ndarray          # int64[nnz]   canonical position -> CSR position
    val: np.ndarray           # float64[nnz] canonical order

    @property
    def col_ptr(self) -> np.ndarray:
        """int32[T, C+1]: start of every local column, relative to the tile's first nonzero."""
        if getattr(self, "_col_ptr", None) is None:
            key = self.tile_of_nnz() * self.C + self.col_local.astype(np.int64)
            q = (np.arange(self.T, dtype=np.int64)[:, None] * self.C
                 + np.arange(self.C + 1, dtype=np.int64)[None, :])
            pos = np.searchsorted(key, q.ravel(), side="left").reshape(self.T, self.C + 1)
            self._col_ptr = (pos - self.tile_nnz_ptr[:-1, None]).astype(np.int32)
        return self._col_ptr

    @property
    def T(self) -> int:
        return int(self.tile_col_idx.size)

    @property
    def nnz(self) -> int:
        return int(self.tile_nnz_ptr[-1])

    def tile_of_nnz(self) -> np.ndarray:
        """Tile index of every canonical nonzero."""
        return np.repeat(np.arange(self.T, dtype=np.int64), np.diff(self.tile_nnz_ptr))

    def tile_row_block(self) -> np.ndarray:
        """Row block of every tile."""
        nrb = self.tile_row_ptr.size - 1
        return np.repeat(np.arange(nrb, dtype=np.int64), np.diff(self.tile_row_ptr))

    def local_col(self) -> np.ndarray:
        """Local column of every canonical nonzero."""
        return self.col_local.astype(np.int64)


def build(n: int, indptr: np.ndarray, indices: np.ndarray, data: np.ndarray,
          R: int, C: int) -> TileCSC:
    """Canonical Tile-CSC of a square CSR matrix (sorted, unique column indices)."""
    if not (1 <= R <= 16384 and 1 <= C <= 256):
        raise ValueError("tile height must lie in [1, 16384] and width in [1, 256]")
    indptr = np.asarray(indptr, dtype=np.int64)
    indices = np.asarray(indices, dtype=np.int64)
    nnz = int(indptr[-1])
    rows = np.repeat(np.arange(n, dtype=np.int64), np.diff(indptr))
    I = rows // R
    J = indices // C
    r = rows - I * R
    c = indices - J * C
    # Canonical order: row block, then column block, then local column, then local row.
    perm = np.lexsort((r, c, J, I))
    I_s, J_s, c_s, r_s = I[perm], J[perm], c[perm], r[perm]
    if nnz:
        new_tile = np.ones(nnz, dtype=bool)
        new_tile[1:] = (I_s[1:] != I_s[:-1]) | (J_s[1:] != J_s[:-1])
        starts = np.nonzero(new_tile)[0]
    else:
        starts = np.zeros(0, dtype=np.int64)
    T = starts.size
    nrb = -(-n // R)
    tile_nnz_ptr = np.append(starts, nnz).astype(np.int64)
    tile_col_idx = J_s[starts].astype(np.int32)
    tiles_per_rb = np.bincount(I_s[starts], minlength=nrb)
    tile_row_ptr = np.zeros(nrb + 1, dtype=np.int64)
    np.cumsum(tiles_per_rb, out=tile_row_ptr[1:])
    return TileCSC(n=n, R=R, C=C, tile_row_ptr=tile_row_ptr, tile_col_idx=tile_col_idx,
                   tile_nnz_ptr=tile_nnz_ptr, row_idx=r_s.astype(np.uint16),
                   col_local=c_s.astype(np.uint8), perm=perm.astype(np.int64),
                   val=np.asarray(data, dtype=np.float64)[perm])


def to_csr(L: TileCSC):
    """Inverse map: rebuild (indptr, indices, data) in CSR order from the tiles."""
    tile = L.tile_of_nnz()
    rb = L.tile_row_block()[tile]
    rows = rb * L.R + L.row_idx.astype(np.int64)
    cols = L.tile_col_idx.astype(np.int64)[tile] * L.C + L.local_col()
    order = np.lexsort((cols, rows))
    indptr = np.zeros(L.n + 1, dtype=np.int64)
    np.cumsum(np.bincount(rows, minlength=L.n), out=indptr[1:])
    return indptr, cols[order], L.val[order]


def padded_columns(L: TileCSC, t: int):
    """Fig. 4(b) view of tile t: every column padded to an even length with sentinel row R.

    Returns (colPtr, rowIdx lists). Storage detail only; the canonical layout
    carries no padding.
    """
    s = int(L.tile_nnz_ptr[t])
    ptr = [0]
    rows = []
    for c in range(L.C):
        a, b = int(L.col_ptr[t, c]), int(L.col_ptr[t, c + 1])
        col = [int(v) for v in L.row_idx[s + a:s + b]]
        if len(col) % 2:
            col.append(L.R)
        rows.append(col)
        ptr.append(ptr[-1] + len(col))
    return ptr, rows


def tile_numbering(n: int, indptr, indices, R: int, C: int):
    """Canonical tile numbers without building the whole layout.

    Returns ``(keys, tile_row_ptr)``: the sorted distinct tile keys
    I * ncb + J (their position is the canonical tile number) and the tile
    row pointers. :func:`tile_of` maps entries to tile numbers with it.
    """
    indptr = np.asarray(indptr, dtype=np.int64)
    ncb = -(-n // C)
    rows = np.repeat(np.arange(n, dtype=np.int64), np.diff(indptr))
    keys = np.unique((rows // R) * ncb + np.asarray(indices, dtype=np.int64) // C)
    nrb = -(-n // R)
    tile_row_ptr = np.zeros(nrb + 1, dtype=np.int64)
    np.cumsum(np.bincount(keys // ncb, minlength=nrb), out=tile_row_ptr[1:])
    return keys, tile_row_ptr


def tile_of(keys, n: int, R: int, C: int, rows, cols):
    """Canonical tile number of entries (rows[i], cols[i]) given :func:`tile_numbering` keys."""
    ncb = -(-n // C)
    k = (np.asarray(rows, dtype=np.int64) // R) * ncb + np.asarray(cols, dtype=np.int64) // C
    t = np.searchsorted(keys, k)
    if np.any(t >= keys.size) or np.any(keys[np.minimum(t, keys.size - 1)] != k):
        raise ValueError("entry outside every non-empty tile")
    return t


def padded_layout(L: TileCSC):
    """The canonical layout with every odd-length local column padded (Fig. 4(b)).

    One sentinel entry is appended to each column holding an odd number of
    nonzeros: row index R, value +0.0. Returns (tile_nnz_ptr int64[T+1],
    row_idx uint16[nnz'], col_local uint8[nnz'], val float64[nnz']), in the
    canonical order with the sentinel last in its column.
    """
    ptr = [0]
    rows, cols, vals = [], [], []
    for t in range(L.T):
        s = int(L.tile_nnz_ptr[t])
        for c in range(L.C):
            a, b = int(L.col_ptr[t, c]), int(L.col_ptr[t, c + 1])
            for k in range(s + a, s + b):
                rows.append(int(L.row_idx[k]))
                cols.append(c)
                vals.append(float(L.val[k]))
            if (b - a) % 2:
                rows.append(L.R)
                cols.append(c)
                vals.append(0.0)
        ptr.append(len(rows))
    return (np.asarray(ptr, dtype=np.int64), np.asarray(rows, dtype=np.uint16),
            np.asarray(cols, dtype=np.uint8), np.asarray(vals, dtype=np.float64))
