"""Matrix builders: seeded, vectorised, canonical CSR (sorted, unique columns).

Every builder returns a :class:`CSR` whose column indices are strictly
increasing inside each row. Values are FP64. Nothing here depends on a tile
shape or a precision map.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass
class CSR:
    """Canonical CSR: ``indptr`` int64[n+1], ``indices`` int32[nnz], ``data`` f64[nnz]."""

    n: int
    indptr: np.ndarray
    indices: np.ndarray
    data: np.ndarray

    @property
    def nnz(self) -> int:
        return int(self.indptr[-1])

    def to_scipy(self):
        import scipy.sparse as sp

        return sp.csr_matrix((self.data, self.indices, self.indptr), shape=(self.n, self.n))

    def matvec(self, x: np.ndarray) -> np.ndarray:
        """Exact-value FP64 product used only to form right-hand sides."""
        return self.to_scipy() @ x


def _stencil_csr(shape, offsets, value_fn):
    """Assemble a structured-grid stencil matrix row by row.

    ``shape`` is the grid shape with the slowest axis first; ``offsets`` is a
    list of integer offset tuples sorted so that the linear column index grows
    with the list position. ``value_fn(k, valid, src_idx, dst_idx)`` returns
    the values of offset ``k`` for the valid (in-domain) rows.
    """
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape))
    coords = np.indices(shape, dtype=np.int32).reshape(len(shape), n)
    strides = [int(np.prod(shape[d + 1:])) for d in range(len(shape))]
    nk = len(offsets)
    valid = np.ones((n, nk), dtype=bool)
    cols = np.empty((n, nk), dtype=np.int64)
    vals = np.zeros((n, nk), dtype=np.float64)
    base = np.arange(n, dtype=np.int64)
    for k, off in enumerate(offsets):
        m = np.ones(n, dtype=bool)
        lin = 0
        for d, o in enumerate(off):
            if o != 0:
                c = coords[d] + o
                m &= (c >= 0) & (c < shape[d])
            lin += o * strides[d]
        valid[:, k] = m
        cols[:, k] = base + lin
        src = np.nonzero(m)[0]
        vals[src, k] = value_fn(k, m, src, src + lin)
    counts = valid.sum(axis=1)
    indptr = np.zeros(n + 1, dtype=np.int64)
    np.cumsum(counts, out=indptr[1:])
    indices = cols[valid].astype(np.int32)
    data = vals[valid]
    return CSR(n, indptr, indices, data)


def _sorted_offsets(dim, radius=1, full=True):
    """All offsets in {-1,0,1}^dim (full) or the 2*dim+1 axis offsets, in column order."""
    if full:
        grids = np.indices((3,) * dim).reshape(dim, -1).T - radius
        offs = [tuple(int(v) for v in g) for g in grids]
    else:
        offs = [tuple(0 for _ in range(dim))]
        for d in range(dim):
            for s in (-1, 1):
                o = [0] * dim
                o[d] = s
                offs.append(tuple(o))
    strides = [3 ** (dim - 1 - d) for d in range(dim)]
    offs.sort(key=lambda o: sum(v * s for v, s in zip(o, strides)))
    return offs


def laplace2d_5pt(m: int) -> CSR:
    """2D 5-point Laplacian on an m x m interior grid, Dirichlet: 4 on the diagonal, -1 off."""
    offs = _sorted_offsets(2, full=False)

    def val(k, mask, src, dst):
        return 4.0 if offs[k] == (0, 0) else -1.0

    return _stencil_csr((m, m), offs, val)


def laplace3d_7pt(m: int) -> CSR:
    """3D 7-point Laplacian on an m^3 interior grid, Dirichlet: 6 on the diagonal, -1 off."""
    offs = _sorted_offsets(3, full=False)

    def val(k, mask, src, dst):
        return 6.0 if offs[k] == (0, 0, 0) else -1.0

    return _stencil_csr((m, m, m), offs, val)


def diffusion3d_27pt(m: int, seed: int = 1) -> CSR:
    """Cell-centred 27-neighbour variable-coefficient diffusion on an m^3 grid.

    Per cell coefficient c_i = 10**U[-3, 3] (``default_rng(seed)``). For a
    neighbour at offset d the geometric weight is g_d = 1/|d|^2 (1, 1/2, 1/3
    for face, edge and corner neighbours) and the coupling is the harmonic
    mean w_ij = g_d * 2 c_i c_j / (c_i + c_j). Off-diagonals are -w_ij. The
    diagonal is the sum of the couplings plus a Dirichlet ghost term g_d*c_i
    for every out-of-domain neighbour, so the matrix is symmetric and
    diagonally dominant (strictly on the boundary): SPD.
    """
    n = m ** 3
    rng = np.random.default_rng(seed)
    c = 10.0 ** rng.uniform(-3.0, 3.0, n)
    offs = _sorted_offsets(3, full=True)
    g = [0.0 if o == (0, 0, 0) else 1.0 / float(sum(v * v for v in o)) for o in offs]
    diag = np.zeros(n, dtype=np.float64)
    centre = offs.index((0, 0, 0))
    # Off-diagonal couplings first (the diagonal accumulates them in offset order).
    off_vals = {}
    shape = (m, m, m)
    coords = np.indices(shape, dtype=np.int32).reshape(3, n)
    strides = [m * m, m, 1]
    for k, o in enumerate(offs):
        if k == centre:
            continue
        msk = np.ones(n, dtype=bool)
        lin = 0
        for d in range(3):
            if o[d] != 0:
                cc = coords[d] + o[d]
                msk &= (cc >= 0) & (cc < m)
            lin += o[d] * strides[d]
        w = np.zeros(n, dtype=np.float64)
        src = np.nonzero(msk)[0]
        ci = c[src]
        cj = c[src + lin]
        w[src] = g[k] * (2.0 * ci * cj) / (ci + cj)
        ghost = ~msk
        w_ghost = np.where(ghost, g[k] * c, 0.0)
        diag += w + w_ghost
        off_vals[k] = -w
    del coords

    def val(k, mask, src, dst):
        if k == centre:
            return diag[src]
        return off_vals[k][src]

    return _stencil_csr(shape, offs, val)


def aniso2d_q1(m: int, kx: float = 1.0, ky: float = 1e-3) -> CSR:
    """Q1 bilinear FEM stiffness of -div(diag(kx, ky) grad u) on an m x m interior grid.

    Unit spacing, homogeneous Dirichlet (boundary nodes eliminated). The
    9-point stencil is kx*s(dx)*t(dy) + ky*t(dx)*s(dy) with s = (-1, 2, -1)
    and t = (1, 4, 1)/6, which is the tensor-product form of the bilinear
    element stiffness. It has four distinct values and is SPD.
    """
    s = {-1: -1.0, 0: 2.0, 1: -1.0}
    t = {-1: 1.0 / 6.0, 0: 4.0 / 6.0, 1: 1.0 / 6.0}
    offs = _sorted_offsets(2, full=True)  # (dy, dx)

    def val(k, mask, src, dst):
        dy, dx = offs[k]
        return kx * s[dx] * t[dy] + ky * t[dx] * s[dy]

    return _stencil_csr((m, m), offs, val)


def _powerlaw_counts(rng, n, alpha, kmax):
    k = np.arange(1, kmax + 1, dtype=np.float64)
    pmf = k ** (-alpha)
    cdf = np.cumsum(pmf)
    cdf /= cdf[-1]
    u = rng.random(n)
    return (np.searchsorted(cdf, u, side="right") + 1).astype(np.int64).clip(1, kmax)


def random_spd_powerlaw(n: int = 4_000_000, seed: int = 1, band: int = 4,
                        alpha: float = 1.7815, kmax: int = 1980,
                        diag_factor: float = 1.05) -> CSR:
    """Random sparse SPD matrix: a band plus power-law extra couplings.

    Structure: every pair with 0 < |i-j| <= ``band`` (8 band neighbours), and
    for each row i, k_i ~ truncated discrete power law P(k) ~ k^-alpha on
    [1, kmax] extra partners drawn uniformly from [0, n) with replacement.
    Pairs are symmetrised as (min, max), self pairs dropped, duplicates and
    band collisions merged. One N(0,1) value per unique pair is mirrored to
    both triangles; the diagonal is ``diag_factor`` times the absolute
    off-diagonal row sum (strict diagonal dominance, hence SPD). With the
    defaults the mean row length is about 30 and the longest row about 2000.
    """
    rng = np.random.default_rng(seed)
    k = _powerlaw_counts(rng, n, alpha, kmax)
    total = int(k.sum())
    rows = np.repeat(np.arange(n, dtype=np.int64), k)
    cols = rng.integers(0, n, size=total, dtype=np.int64)
    a = np.minimum(rows, cols)
    b = np.maximum(rows, cols)
    del rows, cols
    keep = a != b
    keys_extra = a[keep] * n + b[keep]
    del a, b, keep
    band_keys = []
    base = np.arange(n, dtype=np.int64)
    for d in range(1, band + 1):
        i = base[: n - d]
        band_keys.append(i * n + (i + d))
    keys = np.unique(np.concatenate([keys_extra] + band_keys))
    del keys_extra, band_keys
    vals = rng.standard_normal(keys.size)
    lo = keys // n
    hi = keys - lo * n
    del keys
    # Absolute row sums of the off-diagonal part.
    absrow = np.bincount(lo, weights=np.abs(vals), minlength=n) + \
        np.bincount(hi, weights=np.abs(vals), minlength=n)
    diag = diag_factor * absrow
    # CSR assembly by counting: row i holds its lower-triangle partners (pairs
    # with hi = i), then the diagonal, then its upper partners (lo = i). The
    # keys are sorted by (lo, hi), so the upper partners of a row are already
    # consecutive and ascending; a stable sort by hi does the same for the lower.
    m = lo.size
    n_up = np.bincount(lo, minlength=n)
    n_lo = np.bincount(hi, minlength=n)
    indptr = np.zeros(n + 1, dtype=np.int64)
    np.cumsum(n_lo + 1 + n_up, out=indptr[1:])
    nnz = int(indptr[-1])
    indices = np.empty(nnz, dtype=np.int32)
    data = np.empty(nnz, dtype=np.float64)
    seq = np.arange(m, dtype=np.int64)
    up_first = np.cumsum(n_up) - n_up
    pos = indptr[lo] + n_lo[lo] + 1 + (seq - up_first[lo])
    indices[pos] = hi
    data[pos] = vals
    order = np.argsort(hi, kind="stable")
    hi_s = hi[order]
    lo_first = np.cumsum(n_lo) - n_lo
    pos = indptr[hi_s] + (seq - lo_first[hi_s])
    indices[pos] = lo[order]
    data[pos] = vals[order]
    del order, hi_s, pos, seq
    dpos = indptr[:-1] + n_lo
    indices[dpos] = base
    data[dpos] = diag
    return CSR(n, indptr, indices, data)
