"""Pins for the oracle's P1 variant of the SpMV and for the padded layout.

EvoCG's action sets the precision of the vector tile p^(i) with its column
block (Eq. 9, Eq. 10); its reduced-precision values share one scale per
column (Sec. 3.3.2, "Intra-Tile CSC Execution"); its columns are padded to an
even count with sentinel-marked zeros (Sec. 3.3.2, Fig. 4(b)). The pins tie
each to something other than the oracle: an exact rational-arithmetic
rounding written independently, library products on pre-rounded operands,
the exactness of power-of-two scaling, and the Fig. 4(b) example.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.sparse as sp

from oracle import spmv, tilecsc as tc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _random_csr(n, density, seed, scale_exp=0):
    M = sp.random(n, n, density=density, random_state=np.random.RandomState(seed), format="csr")
    M = (M + sp.eye(n, format="csr")).tocsr()
    M.sort_indices()
    rng = np.random.default_rng(seed)
    M.data = rng.standard_normal(M.nnz) * np.ldexp(1.0, rng.integers(-scale_exp, scale_exp + 1, M.nnz))
    return M


def _round_rational(v: float, mbits: int) -> float:
    """Nearest number with mbits significant bits (exponent >= -126), ties to even.

    Exact rational arithmetic, independent of the oracle's frexp/rint route.
    """
    if v == 0.0:
        return 0.0
    F = Fraction(v)
    sign = -1 if F < 0 else 1
    F = abs(F)
    e = F.numerator.bit_length() - F.denominator.bit_length()
    if Fraction(2) ** e > F:
        e -= 1
    while Fraction(2) ** (e + 1) <= F:
        e += 1
    q = Fraction(2) ** (max(e, -126) - (mbits - 1))
    k = F / q
    n = math.floor(k)
    rem = k - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * float(n * q)


def _rounded(v, prec):
    return v if prec == 0 else _round_rational(v, 24 if prec == 1 else 8)


def test_column_scale_exponents_closed_form():
    # columns: max 3.0 -> 2 (0.75 * 4); 1.0 -> 1; 0.5 -> 0; 0.3 -> -1; -5 -> 3; only an explicit zero -> 0
    rows = [0, 1, 0, 1, 2, 3, 4, 5]
    cols = [0, 0, 1, 2, 3, 4, 5, 5]
    vals = [3.0, -1.0, 1.0, 0.5, 0.3, -5.0, 0.0, 0.0]
    M = sp.csr_matrix((vals, (rows, cols)), shape=(6, 6))
    M.sort_indices()
    M.data[:] = [vals[i] for i in np.lexsort((cols, rows))]
    e = spmv.column_scale_exponents(6, M.indptr, M.indices, M.data)
    assert e.tolist() == [2, 1, 0, -1, 3, 0]


def test_column_scale_puts_column_max_in_half_open_unit_interval():
    M = _random_csr(300, 0.03, 4, scale_exp=400)
    e = spmv.column_scale_exponents(300, M.indptr, M.indices, M.data)
    scaled = np.abs(np.ldexp(M.data, -e[M.indices]))
    colmax = np.zeros(300)
    np.maximum.at(colmax, M.indices, scaled)
    assert np.all((colmax >= 0.5) & (colmax < 1.0))


@pytest.mark.parametrize("R,C,seed", [(8, 6, 1), (16, 16, 2), (5, 32, 3)])
def test_p1_without_rounding_or_scale_is_the_plain_product(R, C, seed):
    n = 70
    M = _random_csr(n, 0.08, seed)
    L = tc.build(n, M.indptr, M.indices, M.data, R, C)
    prec = np.random.default_rng(seed).integers(0, 3, L.T).astype(np.uint8)
    x = np.random.default_rng(seed + 1).standard_normal(n)
    a = spmv.spmv_p1_loop(L, M.indptr, M.indices, M.data, prec, x, round_vector=False)
    b = spmv.spmv_loop(L, M.indptr, M.indices, prec, x)
    assert np.array_equal(a, b)


def test_p1_vector_rounding_is_identity_on_bf16_exact_vectors():
    n = 64
    M = _random_csr(n, 0.1, 5)
    L = tc.build(n, M.indptr, M.indices, M.data, 16, 16)
    prec = np.random.default_rng(6).integers(0, 3, L.T).astype(np.uint8)
    x = np.ldexp(np.random.default_rng(7).integers(-128, 128, n).astype(np.float64), -5)
    a = spmv.spmv_p1_loop(L, M.indptr, M.indices, M.data, prec, x, round_vector=True)
    b = spmv.spmv_loop(L, M.indptr, M.indices, prec, x)
    assert np.array_equal(a, b)


def test_p1_fp32_map_equals_product_with_float32_vector():
    n = 90
    M = _random_csr(n, 0.07, 8)
    L = tc.build(n, M.indptr, M.indices, M.data, 16, 16)
    prec = np.ones(L.T, np.uint8)
    x = np.random.default_rng(9).standard_normal(n)
    M32 = M.copy()
    M32.data = M.data.astype(np.float32).astype(np.float64)
    y_ref = M32 @ x.astype(np.float32).astype(np.float64)
    bound = 1e-15 * (abs(M32) @ np.abs(x))
    for y in (spmv.spmv_p1(L, M.indptr, M.indices, M.data, prec, x),
              spmv.spmv_p1_loop(L, M.indptr, M.indices, M.data, prec, x)):
        assert np.all(np.abs(y - y_ref) <= bound)
    # dropping the vector rounding is detected
    y_unrounded = M32 @ x
    assert np.max(np.abs(y_unrounded - y_ref) / (abs(M32) @ np.abs(x))) > 1e-10


def test_p1_bf16_map_matches_torch_on_fp32_exact_operands():
    torch = pytest.importorskip("torch")
    n = 80
    M = _random_csr(n, 0.08, 10)
    M.data = M.data.astype(np.float32).astype(np.float64)
    L = tc.build(n, M.indptr, M.indices, M.data, 16, 16)
    prec = np.full(L.T, 2, np.uint8)
    x = np.random.default_rng(11).standard_normal(n).astype(np.float32).astype(np.float64)

    def bf(v):  # single rounding: the inputs are FP32-exact
        return torch.tensor(np.asarray(v, np.float32)).to(torch.bfloat16).double().numpy()

    Mb = M.copy()
    Mb.data = bf(M.data)
    y_ref = Mb @ bf(x)
    bound = 1e-15 * (abs(Mb) @ np.abs(bf(x)))
    for y in (spmv.spmv_p1(L, M.indptr, M.indices, M.data, prec, x),
              spmv.spmv_p1_loop(L, M.indptr, M.indices, M.data, prec, x)):
        assert np.all(np.abs(y - y_ref) <= bound)


@pytest.mark.parametrize("R,C,seed", [(2, 3, 12), (3, 2, 13), (4, 4, 14)])
def test_p1_mixed_map_matches_exact_rational_brute_force(R, C, seed):
    """Every product rounded by exact rational arithmetic, tile found by (i // R, j // C)."""
    n = 9
    rng = np.random.default_rng(seed)
    D = np.where(rng.random((n, n)) < 0.5, rng.standard_normal((n, n)), 0.0)
    np.fill_diagonal(D, 1.0 + rng.random(n))
    M = sp.csr_matrix(D)
    M.sort_indices()
    L = tc.build(n, M.indptr, M.indices, M.data, R, C)
    prec = rng.integers(0, 3, L.T).astype(np.uint8)
    lookup = {(int(I), int(J)): int(prec[t]) for t, (I, J) in
              enumerate(zip(L.tile_row_block(), L.tile_col_idx))}
    x = rng.standard_normal(n) * 1.7
    exact = []
    for i in range(n):
        s = Fraction(0)
        for j in range(n):
            if D[i, j] != 0.0:
                m = lookup[(i // R, j // C)]
                s += Fraction(_rounded(D[i, j], m)) * Fraction(_rounded(x[j], m))
        exact.append(float(s))
    exact = np.array(exact)
    bound = 1e-15 * (np.abs(D) @ np.abs(x)) + 1e-300
    for y in (spmv.spmv_p1(L, M.indptr, M.indices, M.data, prec, x),
              spmv.spmv_p1_loop(L, M.indptr, M.indices, M.data, prec, x)):
        assert np.all(np.abs(y - exact) <= bound)


def test_p1_column_scale_commutes_with_power_of_two_column_scaling():
    """y(A D, x) = y(A, D x) exactly for D = diag(2^k_j), also far outside FP32's range."""
    n = 60
    M = _random_csr(n, 0.1, 15)
    L = tc.build(n, M.indptr, M.indices, M.data, 8, 8)
    prec = np.random.default_rng(16).integers(0, 3, L.T).astype(np.uint8)
    k = np.random.default_rng(17).integers(-250, 251, n)
    MD = M.copy()
    MD.data = np.ldexp(M.data, k[M.indices])
    LD = tc.build(n, MD.indptr, MD.indices, MD.data, 8, 8)
    x = np.random.default_rng(18).standard_normal(n)
    e = spmv.column_scale_exponents(n, M.indptr, M.indices, M.data)
    eD = spmv.column_scale_exponents(n, MD.indptr, MD.indices, MD.data)
    assert np.array_equal(eD, e + k)
    a = spmv.spmv_p1_loop(LD, MD.indptr, MD.indices, MD.data, prec, x, round_vector=False, col_exp=eD)
    b = spmv.spmv_p1_loop(L, M.indptr, M.indices, M.data, prec, np.ldexp(x, k), round_vector=False, col_exp=e)
    assert np.array_equal(a, b)
    assert np.all(np.isfinite(a))
    # without the scale the FP32 and BF16 entries over- or underflow
    c = spmv.spmv_p1_loop(LD, MD.indptr, MD.indices, MD.data, prec, x, round_vector=False)
    assert not np.allclose(a, c, rtol=1e-2, atol=0.0)


def test_p1_column_scale_is_exact_inside_the_format_range():
    n = 70
    M = _random_csr(n, 0.08, 19, scale_exp=60)
    L = tc.build(n, M.indptr, M.indices, M.data, 16, 16)
    prec = np.random.default_rng(20).integers(0, 3, L.T).astype(np.uint8)
    x = np.random.default_rng(21).standard_normal(n)
    e = spmv.column_scale_exponents(n, M.indptr, M.indices, M.data)
    for rv in (False, True):
        a = spmv.spmv_p1_loop(L, M.indptr, M.indices, M.data, prec, x, round_vector=rv, col_exp=e)
        b = spmv.spmv_p1_loop(L, M.indptr, M.indices, M.data, prec, x, round_vector=rv)
        assert np.array_equal(a, b)


def test_p1_column_scale_keeps_relative_accuracy_beyond_fp32_range():
    """Columns at 1e45 and 1e-48: with the scale every FP32 product is within 2^-24 relative."""
    n = 4
    D = np.diag([3.0e45, 7.0e-48, 1.5, -2.5e45])
    D[0, 1] = 5.0e-48
    M = sp.csr_matrix(D)
    M.sort_indices()
    L = tc.build(n, M.indptr, M.indices, M.data, 4, 4)
    prec = np.ones(L.T, np.uint8)
    x = np.array([1.0, 1.0, 1.0, 1.0])
    e = spmv.column_scale_exponents(n, M.indptr, M.indices, M.data)
    y = spmv.spmv_p1_loop(L, M.indptr, M.indices, M.data, prec, x, col_exp=e)
    exact = D @ x
    assert np.all(np.abs(y - exact) <= 2.0 ** -23 * (np.abs(D) @ np.abs(x)))
    y0 = spmv.spmv_p1_loop(L, M.indptr, M.indices, M.data, prec, x)
    assert np.isinf(y0[0]) and y0[1] == 0.0


def test_padded_layout_reproduces_fig4b():
    g = json.load(open(os.path.join(GOLDEN, "fig4b_intra_tile_csc.json")))
    R, C = g["R"], g["C"]
    n = 2 * C
    rows, cols = [], []
    for c, rs in g["columns"].items():
        rows += rs
        cols += [int(c)] * len(rs)
    M = sp.csr_matrix((np.ones(len(rows)), (rows, cols)), shape=(n, n))
    M.sort_indices()
    L = tc.build(n, M.indptr, M.indices, M.data, R, C)
    ptr, ridx, cloc, val = tc.padded_layout(L)
    t0 = ridx[ptr[0]:ptr[1]]
    c0 = cloc[ptr[0]:ptr[1]]
    colptr = np.searchsorted(c0, np.arange(C + 1))
    assert colptr[:3].tolist() == g["padded_colPtr_head"]
    assert int(colptr[-1]) == g["padded_colPtr_last"]
    for c, expect in g["padded_rowIdx"].items():
        exp = [R - 1 if v == "R-1" else (R if v == "R" else v) for v in expect]
        assert t0[colptr[int(c)]:colptr[int(c) + 1]].tolist() == exp
    assert val[ptr[0] + 3] == 0.0


@pytest.mark.parametrize("R,C,seed", [(16, 16, 22), (7, 5, 23), (32, 32, 24)])
def test_padded_layout_invariants(R, C, seed):
    n = 100
    M = _random_csr(n, 0.06, seed)
    L = tc.build(n, M.indptr, M.indices, M.data, R, C)
    ptr, ridx, cloc, val = tc.padded_layout(L)
    sentinel = ridx == R
    assert np.all(val[sentinel] == 0.0) and not np.any(np.signbit(val[sentinel]))
    # stripping the sentinels gives the canonical layout back
    assert np.array_equal(ridx[~sentinel], L.row_idx.astype(np.uint16))
    assert np.array_equal(cloc[~sentinel], L.col_local)
    assert np.array_equal(val[~sentinel], L.val)
    tile = np.repeat(np.arange(L.T), np.diff(ptr))
    assert np.array_equal(np.bincount(tile[~sentinel], minlength=L.T), np.diff(L.tile_nnz_ptr))
    # every local column even, its sentinel last, at most one per column
    key = tile * C + cloc
    counts = np.bincount(key, minlength=L.T * C)
    assert np.all(counts % 2 == 0)
    s_count = np.bincount(key[sentinel], minlength=L.T * C)
    assert s_count.max(initial=0) <= 1
    last_of_col = np.ones(key.size, bool)
    last_of_col[:-1] = key[1:] != key[:-1]
    assert np.all(last_of_col[sentinel])


def test_p1_fp64_stream_is_not_scaled():
    """A column spanning 1e300 .. 1e-300: FP64 tiles keep the small entry exactly."""
    n = 4
    D = np.diag([1.0e300, 2.0, 3.0, 0.0])
    D[3, 0] = 1.0e-300  # row 3 holds only this entry
    M = sp.csr_matrix(D)
    M.sort_indices()
    L = tc.build(n, M.indptr, M.indices, M.data, 2, 2)
    prec = np.zeros(L.T, np.uint8)
    x = np.array([1.0, 1.0, 1.0, 1.0])
    e = spmv.column_scale_exponents(n, M.indptr, M.indices, M.data)
    y = spmv.spmv_p1_loop(L, M.indptr, M.indices, M.data, prec, x, col_exp=e)
    assert y[3] == 1.0e-300 and y[0] == 1.0e300


def _cfg_small(cfg):
    from gen import make_workload
    w = make_workload(cfg, "small")
    A = w.A
    L = tc.build(A.n, A.indptr, A.indices, A.data, w.R, w.C)
    return w, A, L


@pytest.mark.parametrize("cfg", [2, 3])
def test_p1_cg_with_fp64_map_is_the_plain_fp64_run(cfg):
    """FP64 tiles round nothing and are not scaled: the P1 run equals the plain one bit for bit."""
    from oracle import cg
    w, A, L = _cfg_small(cfg)
    sched = cg.StaticSchedule(np.zeros(L.T, np.uint8))
    a = cg.solve(L, A.indptr, A.indices, A.data, w.b, sched, w.tol, 300, keep_maps=False,
                 round_vector=True, column_scale=True)
    b = cg.solve(L, A.indptr, A.indices, A.data, w.b, sched, w.tol, 300, keep_maps=False)
    assert (a.K, a.status, a.hist) == (b.K, b.status, b.hist)
    assert np.array_equal(a.x, b.x)


@pytest.mark.parametrize("rv,cs", [(True, False), (True, True), (False, True)])
def test_p1_cg_uses_the_p1_product_of_each_direction(rv, cs):
    """Every product inside the P1 CG equals spmv_p1 of the direction it multiplied."""
    from oracle import cg
    from gen import configs
    w, A, L = _cfg_small(3)
    prec = configs.static_map(configs.tile_scores(L.T))
    e = spmv.column_scale_exponents(A.n, A.indptr, A.indices, A.data) if cs else None
    count = [0]

    def hook(k, x, r, p, q, alpha):
        ref = spmv.spmv_p1(L, A.indptr, A.indices, A.data, prec, p, round_vector=rv, col_exp=e)
        assert np.array_equal(q, ref)
        count[0] += 1

    res = cg.solve(L, A.indptr, A.indices, A.data, w.b, cg.StaticSchedule(prec), w.tol, 60, trace=hook,
                   keep_maps=False, round_vector=rv, column_scale=cs)
    assert count[0] == res.K == 60
    if rv:
        # the rounded vector changes the trajectory against the matrix-only product
        plain = cg.solve(L, A.indptr, A.indices, A.data, w.b, cg.StaticSchedule(prec), w.tol, 60,
                         keep_maps=False)
        assert plain.hist != res.hist
