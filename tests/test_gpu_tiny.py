"""GPU parity on the smallest systems: n from 1 to 17 rows, tiles from 1x1 to 256x256 (a single
tile far taller and wider than the matrix), both solve paths (three launches per iteration and
the single-workgroup solve), with and without Jacobi, under a random per-tile map.

Every case checks the exported layout and planes bit for bit, the SpMV on every row
(1e-13 (|A||x|)_i), and a CG solve against the oracle: the status, K within one iteration, the
residual history to 1e-6 down to 1e-8 (below that it is rounding noise once the run converges
exactly) and the iterate's true residual. CG on an n x n SPD system ends within a few
iterations of n, so these runs also cover the stop test on the first iterations and the
padding of odd-length vectors."""

import sys

import numpy as np
import pytest
import scipy.sparse as sp

from oracle import cg as ocg, rounding as ord_, spmv as ospmv, tilecsc as otc

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


def _matrix(n, kind):
    """A small SPD matrix: 'tri' the (-1, 4, -1) tridiagonal, 'dense' a full SPD matrix."""
    if kind == "tri" or n == 1:
        M = sp.diags([np.full(n - 1, -1.0), np.full(n, 4.0), np.full(n - 1, -1.0)], [-1, 0, 1], format="csr")
    else:
        G = np.random.default_rng(n).uniform(-1, 1, (n, n))
        M = sp.csr_matrix(G @ G.T + n * np.eye(n))
    M = M.tocsr()
    M.sort_indices()
    return M.indptr.astype(np.int64), M.indices.astype(np.int32), M.data.astype(np.float64), M


CASES = [(n, kind, R, C) for n in (1, 2, 3, 5, 17) for kind in ("tri", "dense") for (R, C) in
         ((1, 1), (2, 3), (16, 16), (256, 256)) if not (kind == "dense" and n == 1)]


@pytest.mark.parametrize("n,kind,R,C", CASES)
@pytest.mark.parametrize("single_block", [-1, 1])
@pytest.mark.parametrize("jacobi", [False, True])
def test_tiny_system_matches_oracle(n, kind, R, C, single_block, jacobi, dev):
    indptr, indices, data, M = _matrix(n, kind)
    L = mpcg.cg_tilecsc_from_csr(n, indptr, indices, data, R, C)
    Lo = otc.build(n, indptr, indices, data, R, C)
    rng = np.random.default_rng(1000 * n + 10 * R + C)
    m = rng.integers(0, 3, L.T).astype(np.uint8)
    S = mpcg.Solver(L, m, jacobi=jacobi, single_block=single_block)
    log(f"tiny n={n} {kind} R={R} C={C} T={L.T} single_block={single_block} jacobi={jacobi}")

    ex = S.cg_export_layout()
    for name in ("tile_row_ptr", "tile_col_idx", "tile_nnz_ptr", "row_idx"):
        assert np.array_equal(ex[name].astype(np.int64), getattr(Lo, name).astype(np.int64)), name
    assert np.array_equal(ex["col_local"].astype(np.int64), Lo.local_col().astype(np.int64))
    assert np.array_equal(ex["val64"].view(np.uint64), Lo.val.view(np.uint64))
    assert np.array_equal(ex["val32"].view(np.uint32), ord_.to_fp32(Lo.val).view(np.uint32))
    assert np.array_equal(ex["bf16"], ord_.bf16_bits(Lo.val))

    x = rng.uniform(-1, 1, n)
    xd = torch.from_numpy(x).to(dev)
    yd = torch.full_like(xd, float("nan"))
    S.cg_spmv(xd, yd)
    torch.cuda.synchronize()
    y_ref = ospmv.spmv(Lo, indptr, indices, m, x)
    bound = 1e-13 * ospmv.abs_bound(indptr, indices, data, x)
    y = yd.cpu().numpy()
    assert np.all(np.abs(y - y_ref) <= bound), (y, y_ref)

    b = M @ rng.uniform(-1, 1, n)
    tol, maxit = 1e-12, 100
    ref = ocg.solve(Lo, indptr, indices, data, b, ocg.StaticSchedule(m), tol, maxit, jacobi=jacobi,
                    keep_maps=False)
    bd = torch.from_numpy(b).to(dev)
    xs = torch.full_like(bd, float("nan"))
    status, K, hist = S.cg_solve(bd, xs, tol, maxit)
    log(f"  gpu {status} K={K}; oracle {ref.status} K={ref.K}")
    assert status == ref.status
    assert abs(K - ref.K) <= 1
    # The last residuals of an exactly converging run are rounding noise; the history is
    # compared where it stands above it.
    k = min(K, ref.K)
    r = np.asarray(ref.hist[:k])
    sel = r >= 1e-8
    assert np.allclose(hist[:k][sel], r[sel], rtol=1e-6, atol=0)
    assert hist[K] <= tol and ref.hist[ref.K] <= tol
    xh = xs.cpu().numpy()
    assert np.all(np.isfinite(xh))
    tr = np.linalg.norm(b - M @ xh) / np.linalg.norm(b)
    assert tr <= 10 * max(ref.true_residual, 1e-12), (tr, ref.true_residual)
    S.close()


SCHED_CASES = [(n, R, C) for n in (1, 2, 5, 17) for (R, C) in ((1, 1), (16, 16), (256, 256))]


@pytest.mark.parametrize("n,R,C", SCHED_CASES)
@pytest.mark.parametrize("sched", ["tile_rule", "pmag", "ratchet"])
@pytest.mark.parametrize("p1", [0, 3])
def test_tiny_system_schedules_match_oracle(n, R, C, sched, p1, dev):
    """The rules that change the map during a solve (the windowed tile rule, the max|p| rule,
    the residual stages), with and without the paper's SpMV numerics (vector rounding and
    column scale), on the smallest systems: status, K within one and the true residual."""
    indptr, indices, data, M = _matrix(n, "dense" if n > 1 else "tri")
    L = mpcg.cg_tilecsc_from_csr(n, indptr, indices, data, R, C)
    Lo = otc.build(n, indptr, indices, data, R, C)
    rng = np.random.default_rng(7 * n + R + C)
    S = mpcg.Solver(L, p1=p1)
    if sched == "tile_rule":
        scores = rng.uniform(0, 1, L.T) * 10.0 ** rng.integers(-2, 3, L.T)
        S.cg_set_schedule_tile_rule(2, scores, 1e-1, 1e-4)
        rs = ocg.TileRuleSchedule(scores, 2, 1e-1, 1e-4)
    elif sched == "pmag":
        S.cg_set_schedule_pmag(1e-6, 1e-3, period=1)
        rs = ocg.PMagSchedule(Lo.C, Lo.tile_col_idx, 1e-6, 1e-3, 1)
    else:
        S.cg_set_schedule_residual((1e-2, 1e-5), (2, 1, 0))
        rs = ocg.RatchetSchedule((1e-2, 1e-5), (2, 1, 0))
    b = M @ rng.uniform(-1, 1, n)
    tol, maxit = (1e-2 if p1 else 1e-12), 100
    ref = ocg.solve(Lo, indptr, indices, data, b, rs, tol, maxit, keep_maps=False,
                    round_vector=bool(p1 & mpcg.CG_P1_ROUND_VECTOR),
                    column_scale=bool(p1 & mpcg.CG_P1_COLUMN_SCALE))
    bd = torch.from_numpy(b).to(dev)
    xs = torch.full_like(bd, float("nan"))
    status, K, hist = S.cg_solve(bd, xs, tol, maxit)
    log(f"tiny n={n} R={R} C={C} {sched} p1={p1}: gpu {status} K={K}; oracle {ref.status} K={ref.K}")
    assert status == ref.status
    assert abs(K - ref.K) <= 1
    xh = xs.cpu().numpy()
    assert np.all(np.isfinite(xh))
    tr = np.linalg.norm(b - M @ xh) / np.linalg.norm(b)
    assert tr <= 10 * max(ref.true_residual, tol), (tr, ref.true_residual)
    S.close()
