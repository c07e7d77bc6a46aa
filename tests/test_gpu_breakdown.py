"""GPU parity of the breakdown rule on hand-built systems, both solve paths.

A breakdown is p.q <= 0 or a non-finite alpha or beta (reading of the
stopping rules, EvoCG paper Sec. 4.1 and the CG recurrence of Sec. 2.1). A
non-finite alpha stops before the update (K and x unchanged); a non-finite
beta stops after it (the update is counted). The oracle and the library must
agree on the status, K, the history and the iterate.
"""

import sys

import numpy as np
import pytest
import scipy.sparse as sp

from oracle import cg as ocg, tilecsc as otc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
mpcg = pytest.importorskip("mixed_precision_sparse_amd")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    return torch.device("cuda:0")


def _diag_case(d, b):
    M = sp.csr_matrix(np.diag(d))
    M.sort_indices()
    return M, np.asarray(b, dtype=np.float64)


CASES = {
    # p.q = 1e-310 > 0 (subnormal), r.r = 1: alpha overflows -> breakdown before the update
    "alpha_overflow": _diag_case([1e-310, 1.0, 1.0, 1.0], [1.0, 0.0, 0.0, 0.0]),
    # alpha = 1e200 finite, r_new.r_new overflows -> beta = inf after the update
    "beta_overflow": _diag_case([1e-250, 1.0], [1e100, 1.0]),
    # a NaN or an infinity in b: r0 is not finite -> rho_0 = 1, breakdown before the first update
    "b_nan": _diag_case([2.0, 3.0, 4.0, 5.0], [1.0, np.nan, 0.0, 0.0]),
    "b_inf": _diag_case([2.0, 3.0, 4.0, 5.0], [1.0, -np.inf, 0.0, 0.0]),
}


@pytest.mark.parametrize("case", sorted(CASES))
@pytest.mark.parametrize("single_block", [1, -1])
def test_breakdown_matches_oracle(case, single_block, dev):
    M, b = CASES[case]
    n = M.shape[0]
    print(f"breakdown {case} single_block={single_block}", flush=True)
    sys.stdout.flush()
    L = mpcg.cg_tilecsc_from_csr(n, M.indptr.astype(np.int64), M.indices.astype(np.int32), M.data, 4, 4)
    Lo = otc.build(n, M.indptr, M.indices, M.data, 4, 4)
    ref = ocg.solve(Lo, M.indptr, M.indices, M.data, b, ocg.StaticSchedule(np.zeros(Lo.T, np.uint8)), 1e-30, 10)
    S = mpcg.Solver(L, single_block=single_block)
    bd = torch.from_numpy(b).to(dev)
    x = torch.full_like(bd, float("nan"))
    status, K, hist = S.cg_solve(bd, x, 1e-30, 10)
    assert status == ref.status == "breakdown"
    assert K == ref.K
    assert len(hist) == len(ref.hist)
    np.testing.assert_array_equal(hist[:1], ref.hist[:1])
    xs = x.cpu().numpy()
    np.testing.assert_allclose(xs, ref.x, rtol=1e-14, atol=0.0)
    S.close()


@pytest.mark.parametrize("tol, maxit", [(1.0, 10), (1e-30, 0), (0.5, 0)])
@pytest.mark.parametrize("single_block", [1, -1])
def test_non_finite_rhs_follows_the_stopping_order(tol, maxit, single_block, dev):
    """With a non-finite b the tolerance test (rho_0 = 1 <= tol) and the iteration cap come
    first, as in the oracle; only past them does the solve stop as a breakdown."""
    M, b = CASES["b_nan"]
    n = M.shape[0]
    L = mpcg.cg_tilecsc_from_csr(n, M.indptr.astype(np.int64), M.indices.astype(np.int32), M.data, 4, 4)
    Lo = otc.build(n, M.indptr, M.indices, M.data, 4, 4)
    ref = ocg.solve(Lo, M.indptr, M.indices, M.data, b, ocg.StaticSchedule(np.zeros(Lo.T, np.uint8)), tol, maxit)
    S = mpcg.Solver(L, single_block=single_block)
    bd = torch.from_numpy(b).to(dev)
    x = torch.full_like(bd, float("nan"))
    status, K, hist = S.cg_solve(bd, x, tol, maxit)
    assert (status, K) == (ref.status, ref.K) and ref.status in ("converged", "maxit")
    np.testing.assert_array_equal(hist, ref.hist)
    np.testing.assert_array_equal(x.cpu().numpy(), ref.x)
    S.close()

