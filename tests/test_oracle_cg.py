"""Pins for the oracle's CG and Jacobi-PCG.

Each check rests on something outside the oracle: a dense Cholesky solve,
the finite-termination property of CG on a matrix with k distinct
eigenvalues, A-orthogonality of the search directions, orthogonality of the
residuals, agreement of the recurrence residual with the true residual, and
the equivalence of Jacobi-PCG with CG on the symmetrically scaled system.
"""

import math

import numpy as np
import pytest
import scipy.linalg as sla
import scipy.sparse as sp

from gen import make_workload
from oracle import cg, tilecsc as tc


def _csr(M):
    M = sp.csr_matrix(M)
    M.sort_indices()
    return M


def _solve(M, b, tol, maxit, R=4, C=4, jacobi=False, trace=None, prec_map=None, x0=None):
    L = tc.build(M.shape[0], M.indptr, M.indices, M.data, R, C)
    sched = cg.StaticSchedule(np.zeros(L.T, np.uint8) if prec_map is None else prec_map)
    return cg.solve(L, M.indptr, M.indices, M.data, b, sched, tol, maxit, x0=x0,
                    jacobi=jacobi, trace=trace)


def test_cg_matches_dense_cholesky():
    rng = np.random.default_rng(0)
    n = 40
    B = rng.standard_normal((n, n))
    Adense = B @ B.T + n * np.eye(n)
    b = rng.standard_normal(n)
    res = _solve(_csr(Adense), b, 1e-14, 500)
    x_chol = sla.cho_solve(sla.cho_factor(Adense), b)
    assert res.status == "converged"
    assert np.linalg.norm(res.x - x_chol) <= 1e-10 * np.linalg.norm(x_chol)


@pytest.mark.parametrize("k", [1, 3, 7])
def test_cg_terminates_in_k_steps_on_k_distinct_eigenvalues(k):
    n = 200
    eig = np.repeat(np.arange(1, k + 1, dtype=np.float64) * 2.0, -(-n // k))[:n]
    rng = np.random.default_rng(k)
    b = rng.uniform(-1, 1, n)
    res = _solve(_csr(sp.diags(eig)), b, 1e-10, 100)
    assert res.status == "converged"
    assert res.K <= k


def _collect(w, iters=10, jacobi=False):
    A = w.A
    P, X, Rv = [], [], []

    def tr(k, x, r, p, q, alpha):
        if k < iters:
            P.append(p.copy())
            X.append(x.copy())
            Rv.append(r.copy())

    L = tc.build(A.n, A.indptr, A.indices, A.data, w.R, w.C)
    sched = cg.StaticSchedule(np.zeros(L.T, np.uint8))
    res = cg.solve(L, A.indptr, A.indices, A.data, w.b, sched, 1e-12, iters, trace=tr,
                   jacobi=jacobi)
    return A.to_scipy(), P, X, Rv, res


def test_search_directions_are_A_orthogonal():
    w = make_workload(1, "small")
    S, P, _, _, _ = _collect(w)
    ap = [S @ p for p in P]
    norms = [math.sqrt(float(p @ q)) for p, q in zip(P, ap)]
    for i in range(len(P)):
        for j in range(len(P)):
            if i != j:
                assert abs(float(P[i] @ ap[j])) / (norms[i] * norms[j]) < 1e-8


def test_residuals_are_orthogonal():
    w = make_workload(2, "small")
    S, _, _, Rv, _ = _collect(w)
    for i in range(len(Rv)):
        for j in range(i):
            c = abs(float(Rv[i] @ Rv[j])) / (np.linalg.norm(Rv[i]) * np.linalg.norm(Rv[j]))
            assert c < 1e-8


def test_recurrence_residual_tracks_true_residual():
    w = make_workload(1, "small")
    A = w.A
    S = A.to_scipy()
    gaps = []

    def tr(k, x, r, p, q, alpha):
        gaps.append(np.linalg.norm((w.b - S @ x) - r) / np.linalg.norm(w.b))

    L = tc.build(A.n, A.indptr, A.indices, A.data, w.R, w.C)
    res = cg.solve(L, A.indptr, A.indices, A.data, w.b, cg.StaticSchedule(np.zeros(L.T, np.uint8)),
                   w.tol, w.maxit, trace=tr)
    assert res.status == "converged"
    assert max(gaps) < 1e-12
    assert abs(res.true_residual - res.hist[-1] * np.linalg.norm(w.b) / np.linalg.norm(w.b)) < 1e-11


def test_jacobi_pcg_equals_cg_on_scaled_system():
    w = make_workload(3, "small")
    A = w.A
    S = A.to_scipy()
    d = S.diagonal()
    Dm = sp.diags(1.0 / np.sqrt(d))
    Sh = _csr(Dm @ S @ Dm)
    bh = w.b / np.sqrt(d)
    m = 25
    r1 = _solve(S.tocsr(), w.b, 0.0, m, R=16, C=16, jacobi=True)
    r2 = _solve(Sh, bh, 0.0, m, R=16, C=16)
    x_from_scaled = r2.x / np.sqrt(d)
    assert r1.K == r2.K == m
    assert np.linalg.norm(r1.x - x_from_scaled) <= 1e-8 * np.linalg.norm(x_from_scaled)


def test_jacobi_pcg_on_diagonal_matrix_is_one_step():
    d = np.linspace(1.0, 1e4, 300)
    b = np.random.default_rng(0).uniform(-1, 1, 300)
    res = _solve(_csr(sp.diags(d)), b, 1e-12, 10, jacobi=True)
    assert res.K == 1
    assert np.allclose(res.x, b / d, rtol=1e-14)


def test_breakdown_on_indefinite_matrix():
    res = _solve(_csr(np.diag([1.0, -1.0])), np.array([1.0, 1.0]), 1e-10, 10)
    assert res.status == "breakdown" and res.K == 0


def test_overflowing_alpha_stops_before_the_update():
    """p.q > 0 but subnormal: alpha = r.r / p.q overflows. The solve stops with breakdown
    before touching the iterate (K = 0, x = x0, one history entry), which is what the
    library does and what its header promises (x holds the last iterate)."""
    M = _csr(np.diag([1e-310, 1.0, 1.0, 1.0]))
    b = np.array([1.0, 0.0, 0.0, 0.0])
    q = M @ b
    assert 0.0 < float(b @ q) < 2.3e-308 and math.isinf(1.0 / float(b @ q))  # the premise
    res = _solve(M, b, 1e-10, 10)
    assert res.status == "breakdown" and res.K == 0 and res.hist == [1.0]
    assert np.array_equal(res.x, np.zeros(4))
    x0 = np.array([0.0, 0.5, -0.25, 2.0])
    r2 = _solve(M, b + M @ x0, 1e-10, 10, x0=x0)
    assert r2.status == "breakdown" and r2.K == 0 and np.array_equal(r2.x, x0)


def test_non_finite_beta_counts_the_update():
    """A finite alpha with an overflowing r_new.r_new gives a non-finite beta: the update of
    that iteration has been applied, so it is counted (K = 1) before the solve stops."""
    # alpha = (1e200 + 1) / (1e-50 + 1) = 1e200; x = alpha b = (1e300, 1e200) stays finite;
    # r_new = (1e100 (1 - 1e-50), 1 - 1e200), whose square overflows, so beta = inf
    M = _csr(np.diag([1e-250, 1.0]))
    b = np.array([1e100, 1.0])
    res = _solve(M, b, 1e-30, 10)
    assert res.status == "breakdown" and res.K == 1 and len(res.hist) == 2
    assert np.all(np.isfinite(res.x)) and res.x[0] == pytest.approx(1e300, rel=1e-12)


def test_degenerate_inputs():
    M = _csr(np.diag([2.0, 3.0, 4.0]))
    z = _solve(M, np.zeros(3), 1e-10, 10)
    assert z.K == 0 and z.hist == [0.0] and z.status == "converged"
    m0 = _solve(M, np.ones(3), 1e-10, 0)
    assert m0.K == 0 and m0.hist == [1.0] and m0.status == "maxit"
    t1 = _solve(M, np.ones(3), 1.0, 10)
    assert t1.K == 0 and t1.status == "converged"
    xs = np.array([1.0, 2.0, 3.0])
    ex = _solve(M, M @ xs, 1e-10, 10, x0=xs)  # exact initial guess
    assert ex.K == 0 and np.array_equal(ex.x, xs)
    # A NaN or an infinity in b (reading R8 with R6): r0 is not finite, rho_0 = 1; the
    # tolerance test and the cap come first, then the first p.q is not finite: breakdown
    # before any update.
    for bad in (np.nan, np.inf, -np.inf):
        b = np.array([1.0, bad, 0.0])
        nf = _solve(M, b, 1e-10, 10)
        assert nf.status == "breakdown" and nf.K == 0 and nf.hist == [1.0] and not nf.x.any()
        assert _solve(M, b, 1.0, 10).status == "converged"
        assert _solve(M, b, 1e-10, 0).status == "maxit"


def test_integer_stencil_mixed_map_reproduces_fp64_history():
    w = make_workload(2, "small")
    A = w.A
    L = tc.build(A.n, A.indptr, A.indices, A.data, 16, 16)
    mixed = np.random.default_rng(2).integers(0, 3, L.T).astype(np.uint8)
    r64 = cg.solve(L, A.indptr, A.indices, A.data, w.b, cg.StaticSchedule(np.zeros(L.T, np.uint8)),
                   w.tol, w.maxit)
    rmx = cg.solve(L, A.indptr, A.indices, A.data, w.b, cg.StaticSchedule(mixed), w.tol, w.maxit)
    assert r64.hist == rmx.hist and np.array_equal(r64.x, rmx.x)


def test_low_precision_values_raise_true_residual_floor():
    """Eq. (3): a perturbed operator leaves a true-residual gap the recurrence does not see."""
    w = make_workload(3, "small")
    A = w.A
    L = tc.build(A.n, A.indptr, A.indices, A.data, 16, 16)
    r16 = cg.solve(L, A.indptr, A.indices, A.data, w.b,
                   cg.StaticSchedule(np.full(L.T, 2, np.uint8)), 1e-10, 10_000)
    r64 = cg.solve(L, A.indptr, A.indices, A.data, w.b,
                   cg.StaticSchedule(np.zeros(L.T, np.uint8)), 1e-10, 10_000)
    assert r64.status == "converged" and r64.true_residual < 1e-9
    assert r16.true_residual > 100 * r16.hist[-1]


def test_reversed_row_order_is_the_same_product_rounded_differently():
    """reverse_rows sums each row of the product in the opposite order: the exact sum of the
    same terms (integer values: bit for bit), the same value within rounding on real data,
    and a different rounding on rows whose terms cancel."""
    rng = np.random.default_rng(5)
    n = 300
    M = sp.random(n, n, density=0.05, random_state=np.random.RandomState(5), format="csr")
    M = _csr(M + M.T + sp.diags(np.full(n, 40.0)))
    L = tc.build(n, M.indptr, M.indices, M.data, 16, 16)
    m = rng.integers(0, 3, L.T).astype(np.uint8)
    for p1 in (False, True):
        ops = [cg.P1Operator(L, M.indptr, M.indices, M.data, True, True, rev) if p1 else
               cg.PerturbedOperator(L, M.indptr, M.indices, M.data, rev) for rev in (False, True)]
        for op in ops:
            op.set_map(m)
        # Integer-valued data and vector: every partial sum is exact in either order.
        Mi = _csr(sp.csr_matrix((np.round(M.data * 4), M.indices, M.indptr), shape=(n, n)))
        Li = tc.build(n, Mi.indptr, Mi.indices, Mi.data, 16, 16)
        xi = rng.integers(-8, 9, n).astype(np.float64)
        ints = [cg.PerturbedOperator(Li, Mi.indptr, Mi.indices, Mi.data, rev) for rev in (False, True)]
        for op in ints:
            op.set_map(np.zeros(Li.T, np.uint8))
        assert np.array_equal(ints[0] @ xi, ints[1] @ xi)
        x = rng.uniform(-1, 1, n)
        y0, y1 = ops[0] @ x, ops[1] @ x
        bound = 1e-13 * (abs(M) @ np.abs(x))
        assert np.all(np.abs(y0 - y1) <= bound)
        assert np.any(y0 != y1)  # the order did change


def test_reversed_row_order_solve_agrees_on_a_well_conditioned_system():
    rng = np.random.default_rng(6)
    n = 200
    M = sp.random(n, n, density=0.03, random_state=np.random.RandomState(6), format="csr")
    M = _csr(M + M.T + sp.diags(np.full(n, 10.0)))
    L = tc.build(n, M.indptr, M.indices, M.data, 8, 8)
    b = rng.standard_normal(n)
    sched = cg.StaticSchedule(np.zeros(L.T, np.uint8))
    r0 = cg.solve(L, M.indptr, M.indices, M.data, b, sched, 1e-12, 500)
    r1 = cg.solve(L, M.indptr, M.indices, M.data, b, sched, 1e-12, 500, reverse_rows=True)
    assert r0.status == r1.status == "converged" and abs(r0.K - r1.K) <= 1
    k = min(r0.K, r1.K)
    assert np.allclose(r0.hist[:k], r1.hist[:k], rtol=1e-9, atol=0)
    assert np.linalg.norm(r0.x - r1.x) <= 1e-10 * np.linalg.norm(r0.x)
