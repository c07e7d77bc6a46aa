"""Pins of the oracle's CG against an independent textbook implementation.

SciPy's `scipy.sparse.linalg.cg` runs the same Hestenes-Stiefel recurrence
(EvoCG paper, Sec. 2.1, Eq. (1): alpha = r.z / p.q, beta = r_new.z_new / r.z)
and, from x0 = 0, stops on the same unpreconditioned residual test
||r_k|| <= tol ||b|| (strict there, non-strict here: a boundary of measure
zero). Its iteration count is the number of callback calls. With the all-FP64
map the oracle must take the same number of iterations and reach the same
iterate; with a per-tile map it must equal textbook CG on the perturbed
operator, built here independently (tile of entry (i, j) = (i // R, j // C),
tiles numbered in row-block-major, column-ascending order; FP32 tiles hold the
IEEE float32 rounding of each value).
"""

import numpy as np
import pytest
import scipy.sparse as sp
import scipy.sparse.linalg as spla

from gen import make_workload
from oracle import cg as ocg, tilecsc as otc


def _scipy_cg(A, b, tol, maxit, M=None):
    calls = []
    x, info = spla.cg(A, b, x0=np.zeros_like(b), rtol=tol, atol=0.0, maxiter=maxit, M=M,
                      callback=lambda xk: calls.append(1))
    return x, len(calls), info


def _oracle(A, R, C, b, tol, maxit, prec=None, jacobi=False):
    L = otc.build(A.shape[0], A.indptr, A.indices, A.data, R, C)
    m = np.zeros(L.T, np.uint8) if prec is None else prec
    return ocg.solve(L, A.indptr, A.indices, A.data, b, ocg.StaticSchedule(m), tol, maxit, jacobi=jacobi,
                     keep_maps=False), L


@pytest.mark.parametrize("cfg", [1, 2])
def test_fp64_map_equals_textbook_cg(cfg):
    w = make_workload(cfg, "small")
    A = w.A.to_scipy()
    ref, _ = _oracle(A, w.R, w.C, w.b, w.tol, w.maxit)
    x, K, info = _scipy_cg(A, w.b, w.tol, w.maxit)
    assert info == 0 and ref.status == "converged"
    assert abs(ref.K - K) <= 1, (ref.K, K)
    assert np.linalg.norm(ref.x - x) <= 1e-8 * np.linalg.norm(x)


def _random_spd(n, seed):
    """D (S + diag(|S| 1 + 1)) D: symmetric, diagonally dominant before the scaling D =
    diag(10^u), u ~ U[-0.5, 0.5], so SPD, with a diagonal spread that Jacobi undoes."""
    rng = np.random.default_rng(seed)
    B = sp.random(n, n, density=0.02, random_state=np.random.RandomState(seed), format="csr")
    B.data = rng.standard_normal(B.nnz)
    S = (B + B.T).tocsr()
    A0 = S + sp.diags(np.asarray(abs(S).sum(axis=1)).ravel() + 1.0)
    D = sp.diags(10.0 ** rng.uniform(-0.5, 0.5, n))
    A = (D @ A0 @ D).tocsr()
    A.sort_indices()
    return A


def test_jacobi_pcg_equals_textbook_pcg():
    A = _random_spd(400, 11)
    b = A @ np.random.default_rng(0).uniform(-1, 1, A.shape[0])
    ref, _ = _oracle(A, 16, 16, b, 1e-10, 2000, jacobi=True)
    plain, _ = _oracle(A, 16, 16, b, 1e-10, 2000)
    dinv = 1.0 / A.diagonal()
    M = spla.LinearOperator(A.shape, matvec=lambda v: dinv * v)
    x, K, info = _scipy_cg(A, b, 1e-10, 2000, M=M)
    assert info == 0 and ref.status == "converged"
    assert abs(ref.K - K) <= 1, (ref.K, K)
    assert ref.K < plain.K  # the preconditioner is doing something
    assert np.linalg.norm(ref.x - x) <= 1e-8 * np.linalg.norm(x)


def _perturbed(A, R, C, tile_prec):
    """A with the values of FP32 tiles rounded to float32 (tile_prec: 0/1 per canonical tile)."""
    A = A.tocoo()
    ncb = -(-A.shape[1] // C)
    key = (A.row // R).astype(np.int64) * ncb + (A.col // C)
    tiles, tid = np.unique(key, return_inverse=True)  # sorted: row-block-major, columns ascending
    vals = A.data.copy()
    fp32 = tile_prec[tid] == 1
    vals[fp32] = vals[fp32].astype(np.float32).astype(np.float64)
    return sp.csr_matrix((vals, (A.row, A.col)), shape=A.shape), len(tiles)


def test_fp32_tile_map_equals_textbook_cg_on_the_perturbed_operator():
    A = _random_spd(500, 12)
    b = A @ np.random.default_rng(0).uniform(-1, 1, A.shape[0])
    L = otc.build(A.shape[0], A.indptr, A.indices, A.data, 16, 16)
    prec = np.random.default_rng(4).integers(0, 2, L.T).astype(np.uint8)
    Ap, T = _perturbed(A, 16, 16, prec)
    assert T == L.T
    ref = ocg.solve(L, A.indptr, A.indices, A.data, b, ocg.StaticSchedule(prec), 1e-12, 4000, keep_maps=False)
    x, K, info = _scipy_cg(Ap, b, 1e-12, 4000)
    assert info == 0 and ref.status == "converged"
    assert abs(ref.K - K) <= max(1, K // 50), (ref.K, K)
    # The oracle solves the perturbed system, not the exact one: far closer to textbook CG on
    # the perturbed operator than to textbook CG on A.
    x64, _, _ = _scipy_cg(A, b, 1e-12, 4000)
    d_pert, d_exact = np.linalg.norm(ref.x - x), np.linalg.norm(ref.x - x64)
    assert d_pert <= 1e-3 * d_exact, (d_pert, d_exact)
