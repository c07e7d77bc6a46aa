"""GPU parity of handles whose SpMV stages the vector segments in LDS (cg_options.stage_x = 1).

The staged sweep reads every x_j from an LDS copy of the batch's distinct
column blocks instead of gathering it from memory (EvoCG paper, Sec. 3.3.2
"Intra-Tile CSC Execution"). Same bars as the default path: SpMV within
1e-13 * (|A||x|)_i per row against the oracle under FP64, mixed and BF16 maps;
CG iteration counts within 2 % and true residuals within 1e-2 relative.
"""

import sys

import numpy as np
import pytest

from gen import make_workload, static_map, tile_scores
from oracle import cg as ocg, spmv as ospmv, tilecsc as otc

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


@pytest.mark.parametrize("cfg", [1, 2, 3, 5])
def test_staged_spmv_matches_oracle(cfg, dev):
    w = make_workload(cfg, "small")
    A = w.A
    log(f"staged spmv cfg{cfg} small n={A.n}")
    L = mpcg.cg_tilecsc_from_csr(A.n, A.indptr, A.indices, A.data, w.R, w.C)
    Lo = otc.build(A.n, A.indptr, A.indices, A.data, w.R, w.C)
    S = mpcg.Solver(L, stage_x=1, single_block=-1)
    Su = mpcg.Solver(L, single_block=-1)
    rng = np.random.default_rng(31 + cfg)
    maps = [np.zeros(L.T, np.uint8), static_map(tile_scores(L.T, 2), 0.2, 0.3), np.full(L.T, 2, np.uint8),
            rng.integers(0, 3, L.T).astype(np.uint8)]
    for x in (rng.uniform(-1, 1, A.n), rng.standard_normal(A.n) * 10.0 ** rng.integers(-3, 4, A.n)):
        xd = torch.from_numpy(x).to(dev)
        for m in maps:
            S.cg_set_precision_map(m)
            Su.cg_set_precision_map(m)
            y = torch.full_like(xd, float("nan"))
            yu = torch.full_like(xd, float("nan"))
            S.cg_spmv(xd, y)
            Su.cg_spmv(xd, yu)
            torch.cuda.synchronize()
            y_ref = ospmv.spmv(Lo, A.indptr, A.indices, m, x)
            bound = 1e-13 * ospmv.abs_bound(A.indptr, A.indices, A.data, x)
            yh = y.cpu().numpy()
            bad = np.nonzero(~(np.abs(yh - y_ref) <= bound))[0]
            assert bad.size == 0, f"{bad.size} rows out of bound, first {bad[:5]}"
            # the staged sweep accumulates the same products in the same order
            assert np.array_equal(yh, yu.cpu().numpy())
    S.close()
    Su.close()


@pytest.mark.parametrize("cfg,mapkind", [(2, "static"), (3, "magnitude"), (5, "fp64")])
def test_staged_cg_matches_oracle(cfg, mapkind, dev):
    w = make_workload(cfg, "small")
    A = w.A
    log(f"staged CG cfg{cfg} small {mapkind}")
    L = mpcg.cg_tilecsc_from_csr(A.n, A.indptr, A.indices, A.data, w.R, w.C)
    Lo = otc.build(A.n, A.indptr, A.indices, A.data, w.R, w.C)
    S = mpcg.Solver(L, stage_x=1, jacobi=w.jacobi, single_block=-1)
    if mapkind == "static":
        m = static_map(tile_scores(L.T, 2), w.map_spec["frac_bf16"], w.map_spec["frac_fp32"])
        S.cg_set_precision_map(m)
    elif mapkind == "magnitude":
        S.cg_map_from_magnitude(w.map_spec["t_bf16"], w.map_spec["t_fp32"])
        m = S.cg_get_active_map()
    else:
        m = np.zeros(L.T, np.uint8)
        S.cg_set_precision_map(m)
    bd = torch.from_numpy(w.b).to(dev)
    x = torch.zeros_like(bd)
    status, K, hist = S.cg_solve(bd, x, w.tol, min(w.maxit, 3000))
    ref = ocg.solve(Lo, A.indptr, A.indices, A.data, w.b, ocg.StaticSchedule(m), w.tol, min(w.maxit, 3000),
                    jacobi=w.jacobi)
    assert status == ref.status
    assert abs(K - ref.K) <= max(1, int(0.02 * ref.K)), (K, ref.K)
    xs = x.cpu().numpy()
    tr = float(np.linalg.norm(w.b - A.to_scipy() @ xs) / np.linalg.norm(w.b))
    assert abs(max(tr, w.tol) - max(ref.true_residual, w.tol)) <= 1e-2 * max(ref.true_residual, w.tol)
    np.testing.assert_allclose(hist[:20], ref.hist[:20], rtol=1e-6)
    S.close()


def test_staged_tile_rule_solve_equals_unstaged(dev):
    """Under the windowed tile rule the product reads every tile from its precision's plane;
    the staged sweep must still form the same products in the same order, so a staged and an
    unstaged handle run the same solve bit for bit."""
    w = make_workload(5, "small")
    A = w.A
    ms = w.map_spec
    L = mpcg.cg_tilecsc_from_csr(A.n, A.indptr, A.indices, A.data, w.R, w.C)
    runs = []
    for stage in (1, 0):
        S = mpcg.Solver(L, stage_x=stage, single_block=-1)
        S.cg_set_schedule_tile_rule(ms["period"], tile_scores(L.T, 2), ms["hi"], ms["lo"])
        bd = torch.from_numpy(w.b).to(dev)
        x = torch.zeros_like(bd)
        status, K, hist = S.cg_solve(bd, x, w.tol, 300)
        torch.cuda.synchronize()
        runs.append((status, K, np.asarray(hist).copy(), x.cpu().numpy(), S.cg_get_map_trace()[1].copy()))
        S.close()
    (s1, k1, h1, x1, c1), (s0, k0, h0, x0, c0) = runs
    log(f"staged tile rule: K={k1} {s1}, unstaged K={k0} {s0}, {len(c1)} windows")
    assert (s1, k1) == (s0, k0) and np.array_equal(h1, h0) and np.array_equal(x1, x0)
    assert np.array_equal(c1, c0) and len(c1) >= 3
