"""GPU parity of column-sliced handles (cg_options.col_slices).

With S column slices the device keeps the tiles slice by slice and every
slice writes a partial product that is summed afterwards. The canonical
layout, maps and results must not change: the exported layout is compared bit
for bit with the oracle's, the SpMV within 1e-13 * (|A||x|)_i, and CG runs
with the usual bars (iterations within 2 %, true residual within 1e-2).
"""

import math
import sys

import numpy as np
import pytest
import scipy.sparse as sp

from gen import make_workload, static_map, tile_scores
from oracle import cg as ocg, maps as omaps, rounding as ord_, spmv as ospmv, tilecsc as otc

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


def _random(n, density, seed):
    S = sp.random(n, n, density=density, random_state=np.random.RandomState(seed), format="csr")
    S = (S + sp.eye(n, format="csr")).tocsr()
    S.data = np.random.default_rng(seed).standard_normal(S.nnz)
    return _M(S)


def _both(A, R, C):
    return (mpcg.cg_tilecsc_from_csr(A.n, A.indptr, A.indices, A.data, R, C),
            otc.build(A.n, A.indptr, A.indices, A.data, R, C))


def _spmv(S, x, dev):
    xd = torch.from_numpy(x).to(dev)
    yd = torch.full_like(xd, float("nan"))
    S.cg_spmv(xd, yd)
    torch.cuda.synchronize()
    return yd.cpu().numpy()


@pytest.mark.parametrize("slices", [2, 5])
@pytest.mark.parametrize("cfg", [2, 4])
def test_sliced_layout_exports_canonical_order(cfg, slices, dev):
    w = make_workload(cfg, "small")
    L, Lo = _both(w.A, w.R, w.C)
    log(f"sliced layout cfg{cfg} S={slices}")
    S = mpcg.Solver(L, col_slices=slices, jacobi=w.jacobi)
    e = S.cg_export_layout()
    assert np.array_equal(e["tile_row_ptr"], Lo.tile_row_ptr)
    assert np.array_equal(e["tile_col_idx"], Lo.tile_col_idx)
    assert np.array_equal(e["tile_nnz_ptr"], Lo.tile_nnz_ptr)
    assert np.array_equal(e["row_idx"], Lo.row_idx) and np.array_equal(e["col_local"], Lo.col_local)
    assert np.array_equal(e["val64"].view(np.uint64), Lo.val.view(np.uint64))
    assert np.array_equal(e["val32"].view(np.uint32), ord_.to_fp32(Lo.val).view(np.uint32))
    assert np.array_equal(e["bf16"], ord_.bf16_bits(Lo.val))
    S.close()


@pytest.mark.parametrize("slices", [1, 2, 7, 16])
@pytest.mark.parametrize("name", ["cfg2", "cfg4", "random", "ragged"])
def test_sliced_spmv_matches_oracle(name, slices, dev):
    if name.startswith("cfg"):
        w = make_workload(int(name[3:]), "small")
        A, R, C = w.A, w.R, w.C
    elif name == "random":
        A, R, C = _random(3000, 0.003, 51), 16, 16
    else:
        A, R, C = _random(1001, 0.01, 52), 7, 5
    L, Lo = _both(A, R, C)
    prec = np.random.default_rng(slices).integers(0, 3, L.T).astype(np.uint8)
    S = mpcg.Solver(L, precision_map=prec, col_slices=slices)
    assert np.array_equal(S.cg_get_active_map(), prec)
    x = np.random.default_rng(9).uniform(-1, 1, A.n)
    y = _spmv(S, x, dev)
    y_ref = ospmv.spmv(Lo, A.indptr, A.indices, prec, x)
    bound = 1e-13 * ospmv.abs_bound(A.indptr, A.indices, A.data, x)
    bad = np.nonzero(~(np.abs(y - y_ref) <= bound))[0]
    assert bad.size == 0, f"S={slices}: {bad.size} rows out of bound, first {bad[:5]}"
    # a second map on the same handle
    prec2 = static_map(tile_scores(L.T, 2))
    S.cg_set_precision_map(prec2)
    assert np.array_equal(S.cg_get_active_map(), prec2)
    y2 = _spmv(S, x, dev)
    assert np.all(np.abs(y2 - ospmv.spmv(Lo, A.indptr, A.indices, prec2, x)) <= bound)
    S.close()


@pytest.mark.parametrize("slices", [16, 64])
def test_more_slices_than_column_blocks(slices, dev):
    """Slices without any column block (ncb < S) still write their zero partials."""
    A = _random(100, 0.05, 54)  # C = 16: 7 column blocks
    L, Lo = _both(A, 16, 16)
    prec = np.random.default_rng(5).integers(0, 3, L.T).astype(np.uint8)
    S = mpcg.Solver(L, precision_map=prec, col_slices=slices)
    x = np.random.default_rng(6).uniform(-1, 1, A.n)
    y = _spmv(S, x, dev)
    y_ref = ospmv.spmv(Lo, A.indptr, A.indices, prec, x)
    bound = 1e-13 * ospmv.abs_bound(A.indptr, A.indices, A.data, x)
    assert np.all(np.abs(y - y_ref) <= bound)
    e = S.cg_export_layout()
    assert np.array_equal(e["tile_col_idx"], Lo.tile_col_idx) and np.array_equal(e["row_idx"], Lo.row_idx)
    assert np.array_equal(S.cg_get_active_map(), prec)
    S.close()


def test_sliced_spmv_with_paper_numerics(dev):
    A = _random(2000, 0.004, 53)
    L, Lo = _both(A, 16, 16)
    prec = np.random.default_rng(3).integers(0, 3, L.T).astype(np.uint8)
    flags = mpcg.CG_P1_ROUND_VECTOR | mpcg.CG_P1_COLUMN_SCALE | mpcg.CG_P1_PAD_COLUMNS
    S = mpcg.Solver(L, precision_map=prec, p1=flags, col_slices=3)
    x = np.random.default_rng(4).standard_normal(A.n)
    y = _spmv(S, x, dev)
    e = ospmv.column_scale_exponents(A.n, A.indptr, A.indices, A.data)
    y_ref = ospmv.spmv_p1(Lo, A.indptr, A.indices, A.data, prec, x, round_vector=True, col_exp=e)
    bound = ospmv.spmv_p1(Lo, A.indptr, A.indices, np.abs(A.data), prec, np.abs(x), round_vector=True, col_exp=e)
    assert np.all(np.abs(y - y_ref) <= 1e-13 * bound)
    S.close()


def _k_close(K, Kref):
    return abs(K - Kref) <= max(1, math.floor(0.02 * Kref))


def _agree(tr, tr_ref, tol):
    a, b = max(tr, tol), max(tr_ref, tol)
    return abs(a - b) <= 1e-2 * b


@pytest.mark.parametrize("cfg,slices", [(4, 4), (2, 3), (3, 8)])
def test_sliced_cg_matches_oracle(cfg, slices, dev):
    w = make_workload(cfg, "small")
    A = w.A
    L, Lo = _both(A, w.R, w.C)
    S = mpcg.Solver(L, jacobi=w.jacobi, col_slices=slices)
    kind = w.map_spec["kind"]
    if kind == "ratchet":
        S.cg_set_schedule_residual(w.map_spec["thresholds"], w.map_spec["prec"])
        sched = ocg.schedule_for(w.map_spec, Lo)
    else:
        prec = static_map(tile_scores(L.T, 2))
        S.cg_set_precision_map(prec)
        sched = ocg.StaticSchedule(prec)
    ref = ocg.solve(Lo, A.indptr, A.indices, A.data, w.b, sched, w.tol, w.maxit, jacobi=w.jacobi, keep_maps=False)
    bd = torch.from_numpy(w.b).to(dev)
    xd = torch.zeros_like(bd)
    status, K, hist = S.cg_solve(bd, xd, w.tol, w.maxit)
    tr = float(np.linalg.norm(w.b - A.to_scipy() @ xd.cpu().numpy()) / np.linalg.norm(w.b))
    log(f"sliced cg cfg{cfg} S={slices}: gpu {status} K={K} true={tr:.3e}; oracle {ref.status} K={ref.K} "
        f"true={ref.true_residual:.3e}")
    assert status == ref.status
    assert _k_close(K, ref.K), (K, ref.K)
    assert _agree(tr, ref.true_residual, w.tol), (tr, ref.true_residual)
    m = min(K, ref.K, 20)
    assert np.allclose(hist[: m + 1], ref.hist[: m + 1], rtol=1e-6, atol=0)
    ks, counts = S.cg_get_map_trace()
    assert counts.tolist() == [c for (_, c, _) in ref.windows]
    S.close()


def test_sliced_cg_with_initial_guess(dev):
    w = make_workload(2, "small")
    A = w.A
    L, Lo = _both(A, w.R, w.C)
    S = mpcg.Solver(L, col_slices=2)
    x0 = np.random.default_rng(1).uniform(-1, 1, A.n)
    ref = ocg.solve(Lo, A.indptr, A.indices, A.data, w.b, ocg.StaticSchedule(np.zeros(L.T, np.uint8)), w.tol,
                    w.maxit, x0=x0, keep_maps=False)
    bd = torch.from_numpy(w.b).to(dev)
    xd = torch.from_numpy(x0.copy()).to(dev)
    status, K, hist = S.cg_solve(bd, xd, w.tol, w.maxit, x0=xd)
    assert status == ref.status and _k_close(K, ref.K)
    assert np.allclose(hist[:10], ref.hist[:10], rtol=1e-6, atol=0)
    S.close()


@pytest.mark.parametrize("slices", [2, 5])
def test_sliced_handle_runs_every_rule(slices, dev):
    """The magnitude, tile and max|p| rules on a sliced handle: the device works in
    slice order, the maps come back in canonical order equal to the oracle's."""
    w = make_workload(3, "small")
    A = w.A
    L, Lo = _both(A, w.R, w.C)
    S = mpcg.Solver(L, col_slices=slices)
    x = np.random.default_rng(slices).uniform(-1, 1, A.n)
    S.cg_map_from_magnitude(1e-4, 1e-2)
    m = omaps.magnitude_rule(Lo, 1e-4, 1e-2)
    assert np.array_equal(S.cg_get_active_map(), m) and len(set(m.tolist())) >= 2
    y = _spmv(S, x, dev)
    assert np.all(np.abs(y - ospmv.spmv(Lo, A.indptr, A.indices, m, x))
                  <= 1e-13 * ospmv.abs_bound(A.indptr, A.indices, A.data, x))
    s = tile_scores(L.T, 2)
    S.cg_set_schedule_tile_rule(10, s, 1e-3, 1e-6)
    for rho in (1.0, 3e-3, 2e-5, 1e-12):
        S.cg_eval_tile_rule(rho)
        assert np.array_equal(S.cg_get_active_map(), omaps.tile_rule(s, rho, 1e-3, 1e-6)), rho
    S.cg_set_schedule_pmag(1e-3, 1e-1)
    xp = x * 10.0 ** np.random.default_rng(1).integers(-5, 1, -(-A.n // w.C))[np.arange(A.n) // w.C]
    y = _spmv(S, xp, dev)
    m = omaps.pmag_rule(xp, Lo.C, Lo.tile_col_idx, 1e-3, 1e-1)
    assert np.array_equal(S.cg_get_active_map(), m) and len(set(m.tolist())) >= 2
    assert np.all(np.abs(y - ospmv.spmv(Lo, A.indptr, A.indices, m, xp))
                  <= 1e-13 * ospmv.abs_bound(A.indptr, A.indices, A.data, xp))
    S.close()
    with pytest.raises(mpcg.CGError):
        mpcg.Solver(L, col_slices=65)


def test_automatic_slices(dev):
    """col_slices = 0 picks S = ceil(8n / L2 of one XCD) for a matrix whose gathers scatter
    far from the diagonal, and no slices for a banded one; the sliced handle's product
    still matches the oracle's."""
    props = torch.cuda.get_device_properties(0)
    l2 = getattr(props, "L2_cache_size", 0) or (4 << 20)
    n = l2 // 2  # x is 4 L2; near = n / 8 entries
    log(f"L2 of one XCD as reported: {l2} bytes; n = {n}")
    rng = np.random.default_rng(5)
    # six random columns per row: 6/7 (7/8)^2 of the entries lie farther than n / 8 from the diagonal
    rows = np.repeat(np.arange(n), 6)
    cols = rng.integers(0, n, rows.size)
    M = sp.csr_matrix((rng.standard_normal(rows.size), (rows, cols)), shape=(n, n)) + sp.eye(n)
    A = _M(M)
    L = mpcg.cg_tilecsc_from_csr(A.n, A.indptr, A.indices, A.data, 16, 16)
    S = mpcg.Solver(L)
    want = min(64, -(-8 * n // l2))
    assert S.cg_get_options()["col_slices"] == want == 4
    x = rng.uniform(-1, 1, n)
    y = _spmv(S, x, dev)
    Lo = otc.build(A.n, A.indptr, A.indices, A.data, 16, 16)
    m = np.zeros(Lo.T, np.uint8)
    assert np.all(np.abs(y - ospmv.spmv(Lo, A.indptr, A.indices, m, x))
                  <= 1e-13 * ospmv.abs_bound(A.indptr, A.indices, A.data, x))
    S.close()
    assert mpcg.Solver(L, col_slices=1).cg_get_options()["col_slices"] == 1
    # banded: every entry within 8 of the diagonal
    B = _M(sp.diags([np.full(n - abs(k), 1.0 + abs(k)) for k in range(-8, 9)], list(range(-8, 9)), format="csr"))
    LB = mpcg.cg_tilecsc_from_csr(B.n, B.indptr, B.indices, B.data, 16, 16)
    assert mpcg.Solver(LB).cg_get_options()["col_slices"] == 1
