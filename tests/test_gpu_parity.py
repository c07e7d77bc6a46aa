"""GPU parity tests: the HIP path through the C ABI against the CPU oracle.

Bars: layout, maps and value planes bit-exact; SpMV within
1e-13 * (|A||x|)_i per row; CG iteration counts within 2 % and
FP64-recomputed true residuals within 1e-2 relative.
"""

import math
import sys

import numpy as np
import pytest

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


def build_both(w):
    A = w.A
    L = mpcg.cg_tilecsc_from_csr(A.n, A.indptr, A.indices, A.data, w.R, w.C)
    Lo = otc.build(A.n, A.indptr, A.indices, A.data, w.R, w.C)
    return L, Lo


def spmv_check(S, Lo, A, prec, x, dev):
    xd = torch.from_numpy(x).to(dev)
    yd = torch.full_like(xd, float("nan"))
    S.cg_spmv(xd, yd)
    torch.cuda.synchronize()
    y = yd.cpu().numpy()
    y_ref = ospmv.spmv(Lo, A.indptr, A.indices, prec, x)
    bound = 1e-13 * ospmv.abs_bound(A.indptr, A.indices, A.data, x)
    bad = np.nonzero(~(np.abs(y - y_ref) <= bound))[0]
    assert bad.size == 0, f"{bad.size} rows out of bound, first {bad[:5]}: {y[bad[:5]]} vs {y_ref[bad[:5]]}"
    return y


# ---------------------------------------------------------------------------
# Layout and value planes.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_device_layout_and_planes_bit_exact(cfg, dev):
    w = make_workload(cfg, "small")
    log(f"layout/planes cfg{cfg} small n={w.n}")
    L, Lo = build_both(w)
    S = mpcg.Solver(L)
    e = S.cg_export_layout()
    assert np.array_equal(e["tile_row_ptr"], Lo.tile_row_ptr)
    assert np.array_equal(e["tile_col_idx"], Lo.tile_col_idx)
    assert np.array_equal(e["tile_nnz_ptr"], Lo.tile_nnz_ptr)
    assert np.array_equal(e["row_idx"], Lo.row_idx)
    assert np.array_equal(e["col_local"], Lo.col_local)
    assert np.array_equal(e["val64"], Lo.val)
    assert np.array_equal(e["val32"].view(np.uint32), ord_.to_fp32(Lo.val).view(np.uint32))
    assert np.array_equal(e["bf16"], ord_.bf16_bits(Lo.val))
    S.close()


def test_plane_rounding_special_values(dev):
    """Ties, subnormals, overflow edges and signed zeros through the device plane builder."""
    tiny16 = 2.0 ** -133
    vals = [0.0, -0.0, 1.0, -1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -40,
            tiny16, tiny16 / 2, tiny16 * 1.5, 2.0 ** -126, 2.0 ** -149, 2.0 ** -150, 3 * 2.0 ** -150,
            1e-300, -1e-300, 3.3895313892515355e38, 3.4028235677973366e38, 3.4028235677973366e38 * 1.0000001,
            1e300, -1e300, float.fromhex("0x1.fep127") + 2.0 ** 119, np.nextafter(float.fromhex("0x1.fep127") + 2.0 ** 119, 0),
            math.pi, -math.e, 1e-45, 1.401298464324817e-45, 6e-39, 1.1754942e-38]
    rng = np.random.default_rng(3)
    rand = np.ldexp(rng.uniform(0.5, 1.0, 4000), rng.integers(-160, 140, 4000)) * rng.choice([-1, 1], 4000)
    allv = np.concatenate([np.array(vals), rand])
    n = allv.size
    indptr = np.arange(n + 1, dtype=np.int64)
    indices = np.arange(n, dtype=np.int32)
    L = mpcg.cg_tilecsc_from_csr(n, indptr, indices, allv, 16, 16)
    S = mpcg.Solver(L)
    e = S.cg_export_layout()
    Lo = otc.build(n, indptr, indices, allv, 16, 16)
    assert np.array_equal(e["val32"].view(np.uint32), ord_.to_fp32(Lo.val).view(np.uint32))
    assert np.array_equal(e["bf16"], ord_.bf16_bits(Lo.val))
    S.close()


# ---------------------------------------------------------------------------
# SpMV.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_spmv_parity_small(cfg, dev):
    w = make_workload(cfg, "small")
    log(f"spmv cfg{cfg} small n={w.n}")
    A = w.A
    L, Lo = build_both(w)
    S = mpcg.Solver(L)
    rng = np.random.default_rng(cfg)
    x = rng.uniform(-1, 1, A.n)
    maps = {
        "fp64": np.zeros(L.T, np.uint8),
        "fp32": np.ones(L.T, np.uint8),
        "bf16": np.full(L.T, 2, np.uint8),
        "random": rng.integers(0, 3, L.T).astype(np.uint8),
    }
    for name, m in maps.items():
        S.cg_set_precision_map(m)
        spmv_check(S, Lo, A, m, x, dev)
    S.close()


def test_spmv_extreme_vectors(dev):
    w = make_workload(3, "small")
    A = w.A
    L, Lo = build_both(w)
    m = np.random.default_rng(9).integers(0, 3, L.T).astype(np.uint8)
    S = mpcg.Solver(L, m)
    rng = np.random.default_rng(4)
    x = rng.uniform(-1, 1, A.n)
    x[::5] = 0.0
    x[1::7] = 1e150 * rng.uniform(-1, 1, x[1::7].size)
    x[2::11] = 5e-324 * rng.integers(1, 1000, x[2::11].size)
    spmv_check(S, Lo, A, m, x, dev)
    S.close()


def test_spmv_ragged_and_empty_rows(dev):
    import scipy.sparse as sp

    for (n, R, C) in [(1000, 16, 16), (777, 32, 32), (300, 7, 13), (129, 128, 64), (95, 256, 256), (64, 1, 1)]:
        M = sp.random(n, n, density=0.03, random_state=np.random.RandomState(n), format="lil")
        M.setdiag(np.arange(1, n + 1, dtype=float))
        M[n // 3: n // 3 + R + 3, :] = 0
        M = M.tocsr()
        M.sort_indices()
        L = mpcg.cg_tilecsc_from_csr(n, M.indptr, M.indices, M.data, R, C)
        Lo = otc.build(n, M.indptr, M.indices, M.data, R, C)
        m = np.random.default_rng(n).integers(0, 3, L.T).astype(np.uint8)
        S = mpcg.Solver(L, m)
        x = np.random.default_rng(1).uniform(-1, 1, n)
        log(f"spmv ragged n={n} R={R} C={C} T={L.T}")
        spmv_check(S, Lo, M, m, x, dev)
        S.close()


def test_spmv_is_deterministic(dev):
    w = make_workload(4, "small")
    A = w.A
    L, Lo = build_both(w)
    m = np.random.default_rng(1).integers(0, 3, L.T).astype(np.uint8)
    S = mpcg.Solver(L, m)
    xd = torch.from_numpy(np.random.default_rng(2).uniform(-1, 1, A.n)).to(dev)
    y1 = torch.empty_like(xd)
    y2 = torch.empty_like(xd)
    S.cg_spmv(xd, y1)
    S.cg_spmv(xd, y2)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    S.close()


def test_map_switch_equals_fresh_handle(dev):
    """Switching the map on a live handle gives exactly what a handle created with that map gives."""
    w = make_workload(3, "small")
    A = w.A
    L, Lo = build_both(w)
    m1 = np.zeros(L.T, np.uint8)
    m2 = np.random.default_rng(8).integers(0, 3, L.T).astype(np.uint8)
    S = mpcg.Solver(L, m1)
    xd = torch.from_numpy(np.random.default_rng(2).uniform(-1, 1, A.n)).to(dev)
    y1 = torch.empty_like(xd)
    S.cg_set_precision_map(m2)
    S.cg_spmv(xd, y1)
    S2 = mpcg.Solver(L, m2)
    y2 = torch.empty_like(xd)
    S2.cg_spmv(xd, y2)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert np.array_equal(S.cg_get_active_map(), m2)
    S.close()
    S2.close()


# ---------------------------------------------------------------------------
# Map rules.
# ---------------------------------------------------------------------------
def test_magnitude_rule_bit_exact(dev):
    w = make_workload(3, "small")
    L, Lo = build_both(w)
    S = mpcg.Solver(L)
    S.cg_map_from_magnitude(1e-4, 1e-2)
    assert np.array_equal(S.cg_get_active_map(), omaps.magnitude_rule(Lo, 1e-4, 1e-2))
    S.close()


def test_tile_rule_bit_exact(dev):
    w = make_workload(5, "small")
    L, Lo = build_both(w)
    s = tile_scores(L.T, 2)
    S = mpcg.Solver(L)
    S.cg_set_schedule_tile_rule(10, s, 1e-3, 1e-6)
    for rho in (1.0, 0.37, 3e-3, 1e-3, 2e-5, 1e-6, 3e-7, 1e-12):
        S.cg_eval_tile_rule(rho)
        assert np.array_equal(S.cg_get_active_map(), omaps.tile_rule(s, rho, 1e-3, 1e-6)), rho
    S.close()


# ---------------------------------------------------------------------------
# CG at oracle-friendly sizes.
# ---------------------------------------------------------------------------
def _configure(S, w, L, Lo):
    kind = w.map_spec["kind"]
    scores = tile_scores(L.T, 2)
    static = None
    if kind == "static":
        static = static_map(scores, w.map_spec["frac_bf16"], w.map_spec["frac_fp32"])
        S.cg_set_precision_map(static)
    elif kind == "magnitude":
        S.cg_map_from_magnitude(w.map_spec["t_bf16"], w.map_spec["t_fp32"])
    elif kind == "ratchet":
        S.cg_set_schedule_residual(w.map_spec["thresholds"], w.map_spec["prec"])
    elif kind == "tile_rule":
        S.cg_set_schedule_tile_rule(w.map_spec["period"], scores, w.map_spec["hi"], w.map_spec["lo"])
    return ocg.schedule_for(w.map_spec, Lo, scores=scores, static=static)


def _k_close(K, Kref):
    return abs(K - Kref) <= max(1, math.floor(0.02 * Kref))


def _true_res(A, x, b):
    S = A.to_scipy()
    return float(np.linalg.norm(b - S @ x) / np.linalg.norm(b))


def true_residuals_agree(tr, tr_ref, tol, rel=1e-2):
    """Final true residuals agree within ``rel`` after clamping both at the tolerance.

    The stopping rule only guarantees rho_K <= tol; below tol the value
    depends on which iteration crossed it, so residuals pinned there by the
    rule compare equal. Above tol (a residual-gap floor of a mixed map, or an
    iteration cap) the values themselves must agree.
    """
    a, b = max(tr, tol), max(tr_ref, tol)
    return abs(a - b) <= rel * b


# single_block: -1 = the multi-launch solve, 1 = one workgroup where the
# schedule allows it (static maps, residual stages), else the multi-launch one.
@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("which", ["fp64", "mixed"])
@pytest.mark.parametrize("single_block", [-1, 1])
def test_cg_parity_small(cfg, which, single_block, dev):
    w = make_workload(cfg, "small")
    A = w.A
    log(f"cg cfg{cfg} small map={which} single_block={single_block} n={w.n}")
    L, Lo = build_both(w)
    S = mpcg.Solver(L, jacobi=w.jacobi, single_block=single_block)
    if which == "mixed":
        sched = _configure(S, w, L, Lo)
    else:
        sched = ocg.StaticSchedule(np.zeros(L.T, np.uint8))
    ref = ocg.solve(Lo, A.indptr, A.indices, A.data, w.b, sched, w.tol, w.maxit, jacobi=w.jacobi)
    bd = torch.from_numpy(w.b).to(dev)
    xd = torch.zeros_like(bd)
    status, K, hist = S.cg_solve(bd, xd, w.tol, w.maxit)
    x = xd.cpu().numpy()
    log(f"  gpu K={K} {status} rho={hist[-1]:.3e}; oracle K={ref.K} {ref.status} rho={ref.hist[-1]:.3e}")
    assert status == ref.status
    assert _k_close(K, ref.K), (K, ref.K)
    tr = _true_res(A, x, w.b)
    assert true_residuals_agree(tr, ref.true_residual, w.tol), (tr, ref.true_residual)
    m = min(K, ref.K, 20)
    assert np.allclose(hist[: m + 1], ref.hist[: m + 1], rtol=1e-6, atol=0)
    ks, counts = S.cg_get_map_trace()
    if which == "mixed" and w.map_spec["kind"] in ("static", "magnitude"):
        assert ks.tolist() == [0]
        assert counts[0].tolist() == ref.windows[0][1]
    if which == "mixed" and w.map_spec["kind"] == "ratchet":
        assert ks.tolist() == [wk for (wk, _, _) in ref.windows]
        assert counts.tolist() == [c for (_, c, _) in ref.windows]
    if which == "mixed" and w.map_spec["kind"] == "tile_rule":
        # Windows agree while the trajectories agree (rho identical to 1e-9 at the window start).
        for i, (wk, c, _) in enumerate(ref.windows):
            if i >= len(ks) or wk > min(K, ref.K) or abs(hist[wk] - ref.hist[wk]) > 1e-9 * ref.hist[wk]:
                break
            assert ks[i] == wk and counts[i].tolist() == c, (i, wk)
    S.close()


@pytest.mark.parametrize("single_block", [-1, 1])
def test_cg_initial_guess_and_degenerate_cases(single_block, dev):
    w = make_workload(1, "small")
    A = w.A
    L, Lo = build_both(w)
    S = mpcg.Solver(L, single_block=single_block)
    bd = torch.from_numpy(w.b).to(dev)
    # Nonzero initial guess; x may alias x0.
    x0 = np.random.default_rng(1).uniform(-1, 1, A.n)
    xd = torch.from_numpy(x0.copy()).to(dev)
    status, K, hist = S.cg_solve(bd, xd, w.tol, w.maxit, x0=xd)
    ref = ocg.solve(Lo, A.indptr, A.indices, A.data, w.b, ocg.StaticSchedule(np.zeros(L.T, np.uint8)),
                    w.tol, w.maxit, x0=x0)
    assert status == ref.status and _k_close(K, ref.K)
    # maxit = 0, tol >= 1, b = 0.
    xd = torch.zeros_like(bd)
    assert S.cg_solve(bd, xd, w.tol, 0)[:2] == ("maxit", 0)
    st, K, hist = S.cg_solve(bd, xd, 1.0, 10)
    assert (st, K, hist.tolist()) == ("converged", 0, [1.0])
    st, K, hist = S.cg_solve(torch.zeros_like(bd), xd, 1e-10, 10)
    assert (st, K, hist.tolist()) == ("converged", 0, [0.0])
    assert torch.count_nonzero(xd).item() == 0
    S.close()


@pytest.mark.parametrize("single_block", [-1, 1])
def test_cg_vectors_at_8_byte_offsets(single_block, dev):
    """b, x0 and x as views that start 8 bytes into their buffers (odd n, so the
    last entry is the buffer's last double) give the aligned solve's bits."""
    n = 1001  # 1D Laplacian, tridiag(-1, 2, -1)
    ip = np.concatenate([[0], np.cumsum([2] + [3] * (n - 2) + [2])]).astype(np.int64)
    ind = np.concatenate([[0, 1]] + [[i - 1, i, i + 1] for i in range(1, n - 1)] + [[n - 2, n - 1]]).astype(np.int32)
    val = np.concatenate([[2.0, -1.0]] + [[-1.0, 2.0, -1.0]] * (n - 2) + [[-1.0, 2.0]])
    L = mpcg.cg_tilecsc_from_csr(n, ip, ind, val, 16, 16)
    S = mpcg.Solver(L, single_block=single_block)
    rng = np.random.default_rng(5)
    x0 = rng.uniform(-1, 1, n)
    ref_b = torch.from_numpy(rng.uniform(-1, 1, n)).to(dev)
    ref_x0 = torch.from_numpy(x0).to(dev)
    ref_x = torch.zeros_like(ref_b)
    ref = S.cg_solve(ref_b, ref_x, 1e-10, 2000, x0=ref_x0)
    assert ref[0] == "converged"
    bufs = [torch.zeros(n + 1, dtype=torch.float64, device=dev) for _ in range(3)]
    b1, x01, x1 = (t[1:] for t in bufs)
    b1.copy_(ref_b)
    x01.copy_(ref_x0)
    assert all(t.data_ptr() % 16 == 8 for t in (b1, x01, x1))
    got = S.cg_solve(b1, x1, 1e-10, 2000, x0=x01)
    torch.cuda.synchronize()
    log(f"offset vectors single_block={single_block}: {got[0]} K={got[1]}")
    assert got[:2] == ref[:2] and np.array_equal(got[2], ref[2]) and torch.equal(x1, ref_x)
    assert bufs[2][0].item() == 0.0  # nothing written before the view
    S.close()


@pytest.mark.parametrize("single_block", [-1, 1])
def test_cg_breakdown_on_indefinite_matrix(single_block, dev):
    n = 2
    L = mpcg.cg_tilecsc_from_csr(n, np.array([0, 1, 2]), np.array([0, 1], np.int32),
                                 np.array([1.0, -1.0]), 16, 16)
    S = mpcg.Solver(L, single_block=single_block)
    bd = torch.ones(2, dtype=torch.float64, device=dev)
    xd = torch.zeros_like(bd)
    st, K, hist = S.cg_solve(bd, xd, 1e-10, 10)
    assert st == "breakdown" and K == 0
    S.close()


@pytest.mark.parametrize("graph", [0, 1])
@pytest.mark.parametrize("window", [1, 7, 64])
def test_cg_launch_modes_agree(graph, window, dev):
    """Plain launches and graph replay, for several window lengths, give identical results."""
    w = make_workload(2, "small")
    A = w.A
    L, Lo = build_both(w)
    S = mpcg.Solver(L, use_graph=graph, window=window, single_block=-1)
    bd = torch.from_numpy(w.b).to(dev)
    xd = torch.zeros_like(bd)
    st, K, hist = S.cg_solve(bd, xd, w.tol, w.maxit)
    S2 = mpcg.Solver(L, use_graph=0, window=16, single_block=-1)
    x2 = torch.zeros_like(bd)
    st2, K2, hist2 = S2.cg_solve(bd, x2, w.tol, w.maxit)
    torch.cuda.synchronize()
    assert (st, K) == (st2, K2) and np.array_equal(hist, hist2) and torch.equal(xd, x2)
    # A second solve on the same handle reproduces the first bit for bit.
    x3 = torch.zeros_like(bd)
    assert S.cg_solve(bd, x3, w.tol, w.maxit)[1] == K
    torch.cuda.synchronize()
    assert torch.equal(x3, xd)
    S.close()
    S2.close()


def test_tile_rule_window_maps_bit_exact(dev):
    """Every recorded window map of the per-tile rule equals the oracle's, tile by tile,
    while the two trajectories agree (rho at the window start equal to 1e-9 relative)."""
    w = make_workload(5, "small")
    A = w.A
    L, Lo = build_both(w)
    S = mpcg.Solver(L)
    sched = _configure(S, w, L, Lo)
    S.cg_record_window_maps(w.maxit // w.map_spec["period"] + 2)
    ref = ocg.solve(Lo, A.indptr, A.indices, A.data, w.b, sched, w.tol, w.maxit)
    bd = torch.from_numpy(w.b).to(dev)
    xd = torch.zeros_like(bd)
    st, K, hist = S.cg_solve(bd, xd, w.tol, w.maxit)
    maps = S.cg_get_window_maps()
    ks, counts = S.cg_get_map_trace()
    assert len(maps) == len(ks) > 1
    checked = 0
    for i, (wk, c, m) in enumerate(ref.windows):
        if i >= len(ks) or wk > min(K, ref.K) or abs(hist[wk] - ref.hist[wk]) > 1e-9 * ref.hist[wk]:
            break
        assert ks[i] == wk and np.array_equal(maps[i], m), (i, wk)
        assert np.bincount(maps[i], minlength=3).tolist() == counts[i].tolist()
        checked += 1
    log(f"tile rule: {checked} of {len(ks)} window maps compared bit for bit")
    assert checked >= 3
    S.cg_record_window_maps(0)
    S.close()


def test_tile_rule_products_follow_the_map_after_a_solve(dev):
    """In a solve the tile rule changes the map every window and the SpMV reads each
    tile's values from its precision's plane (no repack). Afterwards cg_spmv under the
    final map matches the oracle: with the rule still set, after the schedule is
    cleared (the packed values are stale then, so the product must keep reading the
    planes), and after a new map is uploaded (and repacked)."""
    w = make_workload(5, "small")
    A = w.A
    L, Lo = build_both(w)
    s = tile_scores(L.T, 2)
    S = mpcg.Solver(L)
    bd = torch.from_numpy(w.b).to(dev)
    for maxit in (35, 120, 400):
        S.cg_set_schedule_tile_rule(10, s, w.map_spec["hi"], w.map_spec["lo"])
        xd = torch.zeros_like(bd)
        S.cg_solve(bd, xd, w.tol, maxit)
        ks, counts = S.cg_get_map_trace()
        m = S.cg_get_active_map()
        log(f"tile rule, maxit {maxit}: {len(ks)} windows, final counts {np.bincount(m, minlength=3).tolist()}")
        assert len(ks) >= 2 and len({tuple(c) for c in counts.tolist()}) >= 2  # the map really changed
        x = np.random.default_rng(maxit).uniform(-1, 1, A.n)
        spmv_check(S, Lo, A, m, x, dev)
        S.cg_clear_schedule()
        assert np.array_equal(S.cg_get_active_map(), m)
        spmv_check(S, Lo, A, m, x, dev)
        m2 = np.random.default_rng(maxit + 1).integers(0, 3, L.T).astype(np.uint8)
        S.cg_set_precision_map(m2)
        spmv_check(S, Lo, A, m2, x, dev)
    S.close()


@pytest.mark.parametrize("R", [3, 5, 13])
@pytest.mark.parametrize("rule", ["tile_rule", "pmag"])
def test_cg_odd_row_groups(R, rule, dev):
    """Row groups of an odd number of rows above 64 (odd R; here the small-system sizing,
    about 16 groups): the CG-mode product's p.q must use every row's own p entry. Runs the
    multi-launch path under the tile rule and the max|p| rule against the oracle."""
    import scipy.sparse as sp

    m = 36  # 1296 rows: groups of 27, 17 and 7 row blocks, 81, 85 and 91 rows
    T1 = sp.diags([-1.0, 2.0, -1.0], [-1, 0, 1], shape=(m, m))
    M = (sp.kron(sp.eye(m), T1) + sp.kron(T1, sp.eye(m))).tocsr()
    M.sort_indices()
    n = M.shape[0]
    indptr, indices, data = M.indptr.astype(np.int64), M.indices.astype(np.int32), M.data.astype(np.float64)
    b = M @ np.random.default_rng(R).uniform(-1, 1, n)
    C = 2
    L = mpcg.cg_tilecsc_from_csr(n, indptr, indices, data, R, C)
    Lo = otc.build(n, indptr, indices, data, R, C)
    S = mpcg.Solver(L)  # automatic sizing: one workgroup's row groups
    assert S.cg_get_options()["single_block"] == 1
    if rule == "tile_rule":
        scores = np.random.default_rng(7).uniform(0, 1, L.T) * 10.0 ** np.random.default_rng(8).integers(-2, 3, L.T)
        S.cg_set_schedule_tile_rule(3, scores, 1e-1, 1e-4)
        sched = ocg.TileRuleSchedule(scores, 3, 1e-1, 1e-4)
    else:
        S.cg_set_schedule_pmag(1e-6, 1e-3)
        sched = ocg.PMagSchedule(Lo.C, Lo.tile_col_idx, 1e-6, 1e-3)
    ref = ocg.solve(Lo, indptr, indices, data, b, sched, 1e-10, 500, keep_maps=False)
    bd = torch.from_numpy(b).to(dev)
    xd = torch.zeros_like(bd)
    status, K, hist = S.cg_solve(bd, xd, 1e-10, 500)
    log(f"odd groups R={R} {rule}: gpu {status} K={K}; oracle {ref.status} K={ref.K}")
    assert status == ref.status and _k_close(K, ref.K), (status, K, ref.status, ref.K)
    k = min(K, ref.K, 20)
    assert np.allclose(hist[: k + 1], ref.hist[: k + 1], rtol=1e-6, atol=0)
    S.close()
