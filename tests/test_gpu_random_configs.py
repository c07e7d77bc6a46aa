"""Seeded random configurations against the oracle: random SPD matrices and tile shapes (row
blocks from 1 to 1024 rows, tiles from 1 to 256 columns, odd sizes included), maps and schedules (static map,
magnitude rule, windowed tile rule, max|p| rule, residual ratchet), and handle options
(Jacobi, column slices, vector staging, the single-workgroup solve, the paper's SpMV numerics).
Every case checks the SpMV on every row (1e-13 (|A||x|)_i, or the oracle's own bound with the
paper's numerics) and a CG solve against the oracle: the first 20 residuals to 1e-6 always; for
runs the oracle finishes within 150 iterations also the status, K within 2 % and the true
residual within 1e-2; slower or capped runs, whose end depends on the summation order, must not
end more than ten times behind the oracle's true residual. The cases are drawn once from a
fixed seed."""

import sys

import numpy as np
import pytest
import scipy.sparse as sp

from oracle import cg as ocg, maps as omaps, spmv as ospmv, tilecsc as otc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
mpcg = pytest.importorskip("mixed_precision_sparse_amd")

RV, CS, PAD = mpcg.CG_P1_ROUND_VECTOR, mpcg.CG_P1_COLUMN_SCALE, mpcg.CG_P1_PAD_COLUMNS
SCHEDULES = ("static", "magnitude", "tile_rule", "pmag", "ratchet")
NCASES = 60


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
        self.S = S.tocsr()
        self.S.sort_indices()
        self.n = self.S.shape[0]
        self.indptr = self.S.indptr.astype(np.int64)
        self.indices = self.S.indices.astype(np.int32)
        self.data = self.S.data.astype(np.float64)


def _case(i):
    """One configuration, drawn from its own seed."""
    rng = np.random.default_rng(1000 + i)
    n = int(rng.integers(40, 6000))
    band = int(rng.integers(1, 9))
    rows, cols = [], []
    for d in range(1, band + 1):
        r = np.arange(n - d)
        rows.append(r)
        cols.append(r + d)
    extra = int(rng.integers(0, 4 * n))
    rows.append(rng.integers(0, n, extra))
    cols.append(rng.integers(0, n, extra))
    r = np.concatenate(rows)
    c = np.concatenate(cols)
    keep = r != c
    r, c = r[keep], c[keep]
    if rng.random() < 0.5:
        v = rng.integers(-9, 10, r.size).astype(np.float64)
    else:
        v = rng.standard_normal(r.size) * 10.0 ** rng.integers(-3, 4, r.size)
    U = sp.coo_matrix((v, (r, c)), shape=(n, n)).tocsr()
    U.sum_duplicates()
    M = (U + U.T).tocsr()
    d = 1.1 * np.asarray(abs(M).sum(axis=1)).ravel() + 1.0
    A = _M(M + sp.diags(d))
    R = int(rng.choice([1, 3, 5, 8, 13, 16, 32, 64, 100, 255, 256, 300, 512, 1024]))
    C = int(rng.choice([1, 2, 3, 5, 8, 16, 32, 64, 128, 256]))
    sched = SCHEDULES[i % len(SCHEDULES)]
    p1 = 0
    if rng.random() < 0.35:
        p1 = int(rng.choice([RV, CS, RV | CS, CS | PAD, RV | CS | PAD]))
        if R > 255:
            p1 &= ~PAD
    opts = dict(jacobi=bool(rng.random() < 0.3), col_slices=int(rng.choice([0, 0, 1, 2, 3])),
                stage_x=int(rng.random() < 0.3), single_block=int(rng.choice([-1, 0])), p1=p1)
    x_star = rng.uniform(-1, 1, n)
    b = A.S @ x_star
    return A, R, C, sched, opts, b, rng


def _spmv_ref(Lo, A, prec, x, p1):
    if p1 & (RV | CS):
        e = ospmv.column_scale_exponents(A.n, A.indptr, A.indices, A.data) if p1 & CS else None
        y = ospmv.spmv_p1(Lo, A.indptr, A.indices, A.data, prec, x, round_vector=bool(p1 & RV), col_exp=e)
        bound = 1e-13 * ospmv.spmv_p1(Lo, A.indptr, A.indices, np.abs(A.data), prec, np.abs(x),
                                      round_vector=bool(p1 & RV), col_exp=e)
        return y, bound
    return ospmv.spmv(Lo, A.indptr, A.indices, prec, x), 1e-13 * ospmv.abs_bound(A.indptr, A.indices, A.data, x)


@pytest.mark.parametrize("i", range(NCASES))
def test_random_configuration_matches_oracle(i, dev):
    A, R, C, sched, opts, b, rng = _case(i)
    log(f"case {i}: n={A.n} nnz={A.S.nnz} R={R} C={C} schedule={sched} options={opts}")
    L = mpcg.cg_tilecsc_from_csr(A.n, A.indptr, A.indices, A.data, R, C)
    Lo = otc.build(A.n, A.indptr, A.indices, A.data, R, C)
    S = mpcg.Solver(L, **opts)

    # SpMV under a random static map, every row.
    m = rng.integers(0, 3, L.T).astype(np.uint8)
    S.cg_set_precision_map(m)
    x = rng.uniform(-1, 1, A.n)
    xd = torch.from_numpy(x).to(dev)
    yd = torch.full_like(xd, float("nan"))
    S.cg_spmv(xd, yd)
    torch.cuda.synchronize()
    y_ref, bound = _spmv_ref(Lo, A, m, x, opts["p1"])
    bad = np.nonzero(~(np.abs(yd.cpu().numpy() - y_ref) <= bound))[0]
    assert bad.size == 0, (bad.size, bad[:5].tolist())

    # CG under the case's schedule.
    scores = rng.uniform(0, 1, L.T) * 10.0 ** rng.integers(-2, 3, L.T)
    if sched == "static":
        S.cg_set_precision_map(m)
        ref_sched = ocg.StaticSchedule(m)
    elif sched == "magnitude":
        S.cg_map_from_magnitude(1e-2, 1e-1)
        mm = S.cg_get_active_map()
        ref_map = omaps.magnitude_rule(Lo, 1e-2, 1e-1)
        assert np.array_equal(mm, ref_map)
        ref_sched = ocg.StaticSchedule(ref_map)
    elif sched == "tile_rule":
        S.cg_set_schedule_tile_rule(3, scores, 1e-1, 1e-4)
        ref_sched = ocg.TileRuleSchedule(scores, 3, 1e-1, 1e-4)
    elif sched == "pmag":
        S.cg_set_schedule_pmag(1e-6, 1e-3, period=2)
        ref_sched = ocg.PMagSchedule(Lo.C, Lo.tile_col_idx, 1e-6, 1e-3, 2)
    else:
        S.cg_set_schedule_residual((1e-2, 1e-5), (2, 1, 0))
        ref_sched = ocg.RatchetSchedule((1e-2, 1e-5), (2, 1, 0))
    # With the vector rounded the true residual floors near 1e-3; stop above it.
    tol = 1e-2 if opts["p1"] & RV else 1e-10
    maxit = 400
    ref = ocg.solve(Lo, A.indptr, A.indices, A.data, b, ref_sched, tol, maxit, jacobi=opts["jacobi"],
                    keep_maps=False, round_vector=bool(opts["p1"] & RV), column_scale=bool(opts["p1"] & CS))
    bd = torch.from_numpy(b).to(dev)
    xs = torch.zeros_like(bd)
    status, K, hist = S.cg_solve(bd, xs, tol, maxit)
    tr = float(np.linalg.norm(b - A.S @ xs.cpu().numpy()) / np.linalg.norm(b))
    log(f"  gpu {status} K={K} true={tr:.3e}; oracle {ref.status} K={ref.K} true={ref.true_residual:.3e}")
    k = min(K, ref.K, 20)
    assert np.allclose(hist[: k + 1], ref.hist[: k + 1], rtol=1e-6, atol=0)
    if ref.status == "breakdown":
        assert status == "breakdown"
    elif ref.status == "converged" and ref.K <= 150:
        # A clean run: the bars of the workload tests. Near the tolerance the true residual
        # differs from the recurrence's by a rounding gap that depends on the summation
        # order, so both are clamped at twice the tolerance.
        assert status == ref.status, (status, ref.status)
        assert abs(K - ref.K) <= max(1, int(0.02 * ref.K)), (K, ref.K)
        a, r = max(tr, 2 * tol), max(ref.true_residual, 2 * tol)
        assert abs(a - r) <= 1e-2 * r, (tr, ref.true_residual)
    else:
        # Slow or capped runs under a perturbed operator: K, the final iterate and its true
        # residual depend on the summation order (the design notes' reading R27); the
        # solve must still not end far behind the oracle's.
        assert status in ("converged", "maxit"), status
        assert tr <= 10 * max(ref.true_residual, tol), (tr, ref.true_residual)
    S.close()
