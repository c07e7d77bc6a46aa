"""GPU parity of the single-workgroup CG solve (cg_options.single_block = 1).

One launch of one workgroup runs every iteration. It is compared with the CPU
oracle on the same seeded inputs at the usual bars (iterations within 2 %,
residual history within 1e-6 relative over the first 20 entries, true
residual within 1e-2 relative after clamping at the tolerance) and with the
multi-launch solve. The cases cover odd n, ragged tiles, one- and two-byte
index packing, both accumulator widths (row groups of at most 64 and of up
to 256 rows), mixed per-tile maps, the magnitude rule, the residual stages,
Jacobi, the iteration cap, a 1 x 1 system, repeated solves on one handle, and
a handle too large for the workgroup's LDS copy of p (multi-launch instead).
"""

import math
import sys

import numpy as np
import pytest
import scipy.sparse as sp

from gen import make_workload, static_map, tile_scores
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


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class _M:
    def __init__(self, S):
        S = S.tocsr()
        S.sort_indices()
        self.n = S.shape[0]
        self.indptr = S.indptr.astype(np.int64)
        self.indices = S.indices.astype(np.int32)
        self.data = S.data.astype(np.float64)

    def to_scipy(self):
        return sp.csr_matrix((self.data, self.indices, self.indptr), shape=(self.n, self.n))


def _spd(n, density, seed):
    """Symmetric, strictly diagonally dominant with positive diagonal: SPD."""
    rng = np.random.default_rng(seed)
    B = sp.random(n, n, density=density, random_state=np.random.RandomState(seed), format="csr")
    B.data = rng.standard_normal(B.nnz)
    S = (B + B.T).tocsr()
    d = np.asarray(abs(S).sum(axis=1)).ravel() + 1.0 + rng.uniform(0, 1, n)
    return _M(S + sp.diags(d))


def _k_close(K, Kref):
    return abs(K - Kref) <= max(1, math.floor(0.02 * Kref))


def _agree(tr, tr_ref, tol):
    a, b = max(tr, tol), max(tr_ref, tol)
    return abs(a - b) <= 1e-2 * b


def _true_res(A, x, b):
    return float(np.linalg.norm(b - A.to_scipy() @ x) / np.linalg.norm(b))


@pytest.mark.parametrize("R,C", [(7, 5), (16, 16), (32, 32), (128, 16), (256, 64)])
@pytest.mark.parametrize("jacobi", [False, True])
def test_single_block_random_spd(R, C, jacobi, dev):
    A = _spd(1001, 0.006, 61 + R)
    L = mpcg.cg_tilecsc_from_csr(A.n, A.indptr, A.indices, A.data, R, C)
    Lo = otc.build(A.n, A.indptr, A.indices, A.data, R, C)
    prec = np.random.default_rng(R * C).integers(0, 3, L.T).astype(np.uint8)
    b = A.to_scipy() @ np.random.default_rng(0).uniform(-1, 1, A.n)
    tol, maxit = 1e-9, 2000
    log(f"single block R={R} C={C} jacobi={jacobi} n={A.n} T={L.T}")
    S = mpcg.Solver(L, precision_map=prec, jacobi=jacobi, single_block=1)
    ref = ocg.solve(Lo, A.indptr, A.indices, A.data, b, ocg.StaticSchedule(prec), tol, maxit, jacobi=jacobi,
                    keep_maps=False)
    bd = torch.from_numpy(b).to(dev)
    xd = torch.zeros_like(bd)
    st, K, hist = S.cg_solve(bd, xd, tol, maxit)
    tr = _true_res(A, xd.cpu().numpy(), b)
    log(f"  gpu {st} K={K} true={tr:.3e}; oracle {ref.status} K={ref.K} true={ref.true_residual:.3e}")
    assert st == ref.status
    assert _k_close(K, ref.K), (K, ref.K)
    assert _agree(tr, ref.true_residual, tol), (tr, ref.true_residual)
    m = min(K, ref.K, 20)
    assert np.allclose(hist[: m + 1], ref.hist[: m + 1], rtol=1e-6, atol=0)
    ks, counts = S.cg_get_map_trace()
    assert ks.tolist() == [0] and counts[0].tolist() == np.bincount(prec, minlength=3).tolist()
    S.close()


@pytest.mark.parametrize("jacobi", [False, True])
def test_single_block_residual_stages(jacobi, dev):
    """BF16 until rho <= 1e-3, FP32 until 1e-6, then FP64: stages, trace and history as the oracle's."""
    A = _spd(1001, 0.006, 71)
    L = mpcg.cg_tilecsc_from_csr(A.n, A.indptr, A.indices, A.data, 16, 16)
    Lo = otc.build(A.n, A.indptr, A.indices, A.data, 16, 16)
    b = A.to_scipy() @ np.random.default_rng(0).uniform(-1, 1, A.n)
    thresholds, prec = (1e-3, 1e-6), (2, 1, 0)
    S = mpcg.Solver(L, jacobi=jacobi, single_block=1)
    S.cg_set_schedule_residual(thresholds, prec)
    ref = ocg.solve(Lo, A.indptr, A.indices, A.data, b, ocg.RatchetSchedule(thresholds, prec), 1e-10, 2000,
                    jacobi=jacobi, keep_maps=False)
    bd = torch.from_numpy(b).to(dev)
    xd = torch.zeros_like(bd)
    st, K, hist = S.cg_solve(bd, xd, 1e-10, 2000)
    tr = _true_res(A, xd.cpu().numpy(), b)
    log(f"stages jacobi={jacobi}: gpu {st} K={K} true={tr:.3e}; oracle {ref.status} K={ref.K}")
    assert st == ref.status and _k_close(K, ref.K), (K, ref.K)
    assert _agree(tr, ref.true_residual, 1e-10)
    m = min(K, ref.K, 20)
    assert np.allclose(hist[: m + 1], ref.hist[: m + 1], rtol=1e-6, atol=0)
    ks, counts = S.cg_get_map_trace()
    assert ks.tolist() == [wk for (wk, _, _) in ref.windows]
    assert counts.tolist() == [c for (_, c, _) in ref.windows]
    assert len(ks) == 3
    S.close()


def test_single_block_beyond_the_lds_copy_runs_multi_launch(dev):
    """A forced handle larger than the LDS copy of p solves on the multi-launch path."""
    from gen.matrices import laplace2d_5pt
    A = laplace2d_5pt(128)  # n = 16384
    L = mpcg.cg_tilecsc_from_csr(A.n, A.indptr, A.indices, A.data, 16, 16)
    Lo = otc.build(A.n, A.indptr, A.indices, A.data, 16, 16)
    b = A.to_scipy() @ np.random.default_rng(0).uniform(-1, 1, A.n)
    ref = ocg.solve(Lo, A.indptr, A.indices, A.data, b, ocg.StaticSchedule(np.zeros(L.T, np.uint8)), 1e-8, 2000,
                    keep_maps=False)
    bd = torch.from_numpy(b).to(dev)
    res = []
    for sb in (1, -1):
        S = mpcg.Solver(L, single_block=sb)
        xd = torch.zeros_like(bd)
        res.append(S.cg_solve(bd, xd, 1e-8, 2000))
        torch.cuda.synchronize()
        S.close()
    (st1, K1, h1), (st2, K2, h2) = res
    assert (st1, K1) == (st2, K2) == (ref.status, K1) and _k_close(K1, ref.K)
    assert np.array_equal(h1, h2)


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_single_block_agrees_with_multi_launch(cfg, dev):
    w = make_workload(cfg, "small")
    A = w.A
    L = mpcg.cg_tilecsc_from_csr(A.n, A.indptr, A.indices, A.data, w.R, w.C)
    res = []
    for sb in (1, -1):
        S = mpcg.Solver(L, jacobi=w.jacobi, single_block=sb)
        if w.map_spec["kind"] == "ratchet":
            S.cg_set_schedule_residual(w.map_spec["thresholds"], w.map_spec["prec"])
        elif w.map_spec["kind"] == "static":
            S.cg_set_precision_map(static_map(tile_scores(L.T, 2)))
        elif w.map_spec["kind"] == "magnitude":
            S.cg_map_from_magnitude(w.map_spec["t_bf16"], w.map_spec["t_fp32"])
        bd = torch.from_numpy(w.b).to(dev)
        xd = torch.zeros_like(bd)
        st, K, hist = S.cg_solve(bd, xd, w.tol, w.maxit)
        ks, counts = S.cg_get_map_trace()
        res.append((st, K, hist, xd.cpu().numpy(), ks.tolist(), counts.tolist()))
        S.close()
    (st1, K1, h1, x1, k1, c1), (st2, K2, h2, x2, k2, c2) = res
    log(f"cfg{cfg}: single block {st1} K={K1}; multi-launch {st2} K={K2}")
    # Summation orders differ between the paths: the usual bars, not bits.
    assert st1 == st2 and _k_close(K1, K2), (K1, K2)
    m = min(K1, K2, 20)
    assert np.allclose(h1[: m + 1], h2[: m + 1], rtol=1e-6, atol=0)
    assert k1 == k2 and c1 == c2
    assert _agree(_true_res(A, x1, w.b), _true_res(A, x2, w.b), w.tol)


def test_single_block_cap_repeat_and_tiny(dev):
    w = make_workload(2, "small")
    A = w.A
    L = mpcg.cg_tilecsc_from_csr(A.n, A.indptr, A.indices, A.data, w.R, w.C)
    Lo = otc.build(A.n, A.indptr, A.indices, A.data, w.R, w.C)
    S = mpcg.Solver(L, single_block=1)
    bd = torch.from_numpy(w.b).to(dev)
    # The iteration cap: 7 iterations, history as the oracle's.
    xd = torch.zeros_like(bd)
    st, K, hist = S.cg_solve(bd, xd, w.tol, 7)
    ref = ocg.solve(Lo, A.indptr, A.indices, A.data, w.b, ocg.StaticSchedule(np.zeros(L.T, np.uint8)), w.tol, 7,
                    keep_maps=False)
    assert (st, K) == ("maxit", 7) == (ref.status, ref.K)
    assert np.allclose(hist, ref.hist, rtol=1e-9, atol=0)
    # Two full solves on one handle give the same bits.
    x1 = torch.zeros_like(bd)
    r1 = S.cg_solve(bd, x1, w.tol, w.maxit)
    x2 = torch.zeros_like(bd)
    r2 = S.cg_solve(bd, x2, w.tol, w.maxit)
    torch.cuda.synchronize()
    assert r1[:2] == r2[:2] and np.array_equal(r1[2], r2[2]) and torch.equal(x1, x2)
    S.close()
    # A 1 x 1 system: one iteration, x = b / a.
    L1 = mpcg.cg_tilecsc_from_csr(1, np.array([0, 1]), np.array([0], np.int32), np.array([4.0]), 16, 16)
    S1 = mpcg.Solver(L1, single_block=1)
    b1 = torch.full((1,), 3.0, dtype=torch.float64, device=dev)
    x1 = torch.zeros_like(b1)
    st, K, hist = S1.cg_solve(b1, x1, 1e-12, 10)
    assert (st, K) == ("converged", 1) and x1.item() == 0.75 and hist.tolist() == [1.0, 0.0]
    S1.close()
    with pytest.raises(mpcg.CGError):
        mpcg.Solver(L1, single_block=2)
