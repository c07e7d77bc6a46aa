"""GPU parity of the per-segment max|p| rule (EvoCG paper, Sec. 4.7) against the oracle.

The rule's decisions are exact on both sides (a maximum of absolute values,
compared in FP64), so for a given vector the map must match bit for bit; the
SpMV then meets the usual 1e-13 * (|A||x|)_i bound. Inside CG the direction
vectors of the two sides differ by rounding, so a column block whose maximum
sits on a threshold may be classified differently once the trajectories have
drifted: per-iteration precision counts are compared while the residual
histories agree, as for the windowed tile rule.
"""

import math
import sys

import numpy as np
import pytest
import scipy.sparse as sp

from gen import make_workload
from oracle import cg as ocg, maps as omaps, spmv as ospmv, tilecsc as otc

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


def _random_spd(n, density, seed, R, C):
    rng = np.random.default_rng(seed)
    M = sp.random(n, n, density=density, random_state=np.random.RandomState(seed), format="csr")
    M = (M + M.T).tocsr()
    M = (M + sp.diags(np.abs(M).sum(axis=1).A1 + 1.0)).tocsr()
    M.sort_indices()
    return M


# Beyond the workloads: C12 (segments of 12 entries, 16-byte loads of 6 pairs),
# C128 (the largest column blocks, a short last one), C8odd (n odd: the last
# column block is short and ends on a single entry) and C7 (odd C and R: the
# segments are read entry by entry).
CASES = [("cfg2", None), ("cfg3", None), ("cfg5", None), ("C12", (300, 0.02, 8, 12)), ("C128", (700, 0.01, 64, 128)),
         ("C8odd", (301, 0.03, 8, 8)), ("C7", (257, 0.03, 9, 7))]


def _case(name, spec):
    if spec is None:
        w = make_workload(int(name[3:]), "small")
        return w.A.n, w.A.indptr, w.A.indices, w.A.data, w.R, w.C
    n, dens, R, C = spec
    M = _random_spd(n, dens, 5, R, C)
    return n, M.indptr.astype(np.int64), M.indices.astype(np.int32), M.data, R, C


@pytest.mark.parametrize("name,spec", CASES)
def test_pmag_spmv_and_map_match_oracle(name, spec, dev):
    n, ip, ind, val, R, C = _case(name, spec)
    log(f"pmag spmv {name} n={n} R={R} C={C}")
    L = mpcg.cg_tilecsc_from_csr(n, ip, ind, val, R, C)
    Lo = otc.build(n, ip, ind, val, R, C)
    S = mpcg.Solver(L)
    rng = np.random.default_rng(11)
    lo, hi = 1e-4, 1e-2
    S.cg_set_schedule_pmag(lo, hi)
    ncb = -(-n // C)
    for trial in range(3):
        # Every column block gets its own scale (FP64, FP32 and BF16 classes in
        # turn); one block's maximum is planted exactly on lo (FP32 by the rule)
        # and one exactly on hi (FP64).
        scale = np.array([1.0, 1e-3, 1e-5])[(np.arange(ncb) + trial) % 3]
        x = rng.uniform(-1, 1, n) * np.repeat(scale, C)[:n]
        J_lo = int(np.nonzero(scale == 1e-5)[0][0])
        J_hi = int(np.nonzero(scale == 1e-3)[0][0])
        x[J_lo * C] = lo
        x[J_hi * C] = -hi
        ref_map = omaps.pmag_rule(x, C, Lo.tile_col_idx, lo, hi)
        xd = torch.from_numpy(x).to(dev)
        yd = torch.full_like(xd, float("nan"))
        S.cg_spmv(xd, yd)
        torch.cuda.synchronize()
        assert np.array_equal(S.cg_get_active_map(), ref_map)
        y_ref = ospmv.spmv(Lo, ip, ind, ref_map, x)
        bound = 1e-13 * ospmv.abs_bound(ip, ind, val, x)
        assert np.all(np.abs(yd.cpu().numpy() - y_ref) <= bound)
        if trial == 0:
            assert set(np.unique(ref_map)) == {0, 1, 2}
    S.close()


@pytest.mark.parametrize("C", [8, 16])
def test_pmag_map_independent_of_vector_alignment(C, dev):
    """x at an 8-byte offset (scalar loads) and at 16-byte offsets (pairs) gives the
    oracle's map; a NaN makes its column block FP64."""
    n, ip, ind, val, R, _ = _case("x", (333, 0.03, 8, C))
    L = mpcg.cg_tilecsc_from_csr(n, ip, ind, val, R, C)
    Lo = otc.build(n, ip, ind, val, R, C)
    S = mpcg.Solver(L)
    lo, hi = 1e-4, 1e-2
    S.cg_set_schedule_pmag(lo, hi)
    ncb = -(-n // C)
    rng = np.random.default_rng(3)
    scale = np.array([1.0, 1e-3, 1e-5])[np.arange(ncb) % 3]
    x = rng.uniform(-1, 1, n) * np.repeat(scale, C)[:n]
    x[2 * C + 1] = np.nan  # block 2 is a BF16 block by scale
    ref_map = omaps.pmag_rule(x, C, Lo.tile_col_idx, lo, hi)
    assert ref_map[Lo.tile_col_idx == 2].tolist() == [0] * int(np.sum(Lo.tile_col_idx == 2))
    buf = torch.zeros(n + 2, dtype=torch.float64, device=dev)
    for off in (1, 2, 0):
        xd = buf[off:off + n]
        xd.copy_(torch.from_numpy(x))
        log(f"pmag alignment C={C} offset {8 * off} bytes, address % 16 = {xd.data_ptr() % 16}")
        yd = torch.empty(n, dtype=torch.float64, device=dev)
        S.cg_spmv(xd, yd)
        torch.cuda.synchronize()
        assert np.array_equal(S.cg_get_active_map(), ref_map), off
    S.close()


@pytest.mark.parametrize("cfg", [2, 3])
def test_pmag_reduces_to_static_maps_bit_for_bit(cfg, dev):
    """lo = hi = 0 is the FP64 map and lo = hi = inf the BF16 map, on the GPU as well."""
    w = make_workload(cfg, "small")
    A = w.A
    L = mpcg.cg_tilecsc_from_csr(A.n, A.indptr, A.indices, A.data, w.R, w.C)
    bd = torch.from_numpy(w.b).to(dev)
    for lo, code in ((0.0, 0), (math.inf, 2)):
        S1 = mpcg.Solver(L)
        S1.cg_set_schedule_pmag(lo, lo)
        x1 = torch.zeros_like(bd)
        st1, K1, h1 = S1.cg_solve(bd, x1, w.tol, 400)
        # The same multi-launch kernels (a small static-map handle could
        # otherwise solve on one workgroup, with another summation order).
        S2 = mpcg.Solver(L, np.full(L.T, code, np.uint8), single_block=-1)
        x2 = torch.zeros_like(bd)
        st2, K2, h2 = S2.cg_solve(bd, x2, w.tol, 400)
        log(f"cfg{cfg} pmag lo=hi={lo}: {st1} K={K1}; static code {code}: {st2} K={K2}")
        assert (st1, K1) == (st2, K2)
        assert np.array_equal(h1, h2)
        assert torch.equal(x1, x2)
        ks, counts = S1.cg_get_map_trace()
        assert ks.tolist() == list(range(K1))  # one entry per iteration run
        assert all(c[code] == L.T for c in counts)
        S1.close()
        S2.close()


@pytest.mark.parametrize("cfg,lo,hi", [(2, 1e-4, 1e-2), (3, 1e-3, 1e-1)])
def test_pmag_cg_matches_oracle(cfg, lo, hi, dev):
    w = make_workload(cfg, "small")
    A = w.A
    L = mpcg.cg_tilecsc_from_csr(A.n, A.indptr, A.indices, A.data, w.R, w.C)
    Lo = otc.build(A.n, A.indptr, A.indices, A.data, w.R, w.C)
    maxit = 10000
    ref = ocg.solve(Lo, A.indptr, A.indices, A.data, w.b, ocg.PMagSchedule(Lo.C, Lo.tile_col_idx, lo, hi),
                    w.tol, maxit, keep_maps=False)
    S = mpcg.Solver(L)
    S.cg_set_schedule_pmag(lo, hi)
    bd = torch.from_numpy(w.b).to(dev)
    xd = torch.zeros_like(bd)
    status, K, hist = S.cg_solve(bd, xd, w.tol, maxit)
    x = xd.cpu().numpy()
    tr = float(np.linalg.norm(w.b - A.to_scipy() @ x) / np.linalg.norm(w.b))
    log(f"cfg{cfg} pmag: GPU {status} K={K} true={tr:.3e}; oracle {ref.status} K={ref.K} "
        f"true={ref.true_residual:.3e}")
    assert status == ref.status
    assert abs(K - ref.K) <= max(1, math.floor(0.02 * ref.K))
    a, b = max(tr, w.tol), max(ref.true_residual, w.tol)
    assert abs(a - b) <= 1e-2 * b
    ks, counts = S.cg_get_map_trace()
    agree = 0
    for k in range(min(K, ref.K)):
        if abs(hist[k] - ref.hist[k]) > 1e-9 * ref.hist[k]:
            break
        assert ks[k] == k and counts[k].tolist() == ref.windows[k][1], k
        agree += 1
    log(f"cfg{cfg} pmag: {agree} of {ref.K} iterations' maps compared while trajectories agree")
    assert agree >= 5
    assert sum(c[1] + c[2] for _, c, _ in ref.windows) > 0  # the rule did lower some tiles
    S.close()


def test_recorded_column_codes_and_kstar_match_oracle(dev):
    """A per-iteration run's recorded column-block codes equal the oracle's while the
    trajectories agree; K* from the recorded codes matches the oracle's selection."""
    w = make_workload(2, "small")
    A = w.A
    lo, hi = 1e-4, 1e-2
    L = mpcg.cg_tilecsc_from_csr(A.n, A.indptr, A.indices, A.data, w.R, w.C)
    Lo = otc.build(A.n, A.indptr, A.indices, A.data, w.R, w.C)
    rec = []
    ref = ocg.solve(Lo, A.indptr, A.indices, A.data, w.b,
                    ocg.PMagSchedule(Lo.C, Lo.tile_col_idx, lo, hi, 1, rec), w.tol, 1000, keep_maps=False)
    S = mpcg.Solver(L)
    S.cg_set_schedule_pmag(lo, hi, 1)
    S.cg_record_column_codes(True)
    bd = torch.from_numpy(w.b).to(dev)
    xd = torch.zeros_like(bd)
    status, K, hist = S.cg_solve(bd, xd, w.tol, 1000)
    codes = S.cg_get_column_codes()
    log(f"pmag record: GPU K={K} records={codes.shape}; oracle K={ref.K} records={len(rec)}")
    assert codes.shape == (K, -(-A.n // w.C))
    agree = 0
    for k in range(min(K, ref.K)):
        if abs(hist[k] - ref.hist[k]) > 1e-9 * ref.hist[k]:
            break
        assert np.array_equal(codes[k], rec[k]), k
        agree += 1
    assert agree >= 5
    kstar, table = mpcg.cg_select_reuse_interval(codes)
    k_ref, table_ref = omaps.select_reuse_interval(codes)
    assert (kstar, [i for i, _ in table]) == (k_ref, [i for i, _ in table_ref])
    if agree == K == ref.K:
        assert kstar == omaps.select_reuse_interval(np.array(rec))[0]
    log(f"pmag record: K*={kstar}, table {table}")
    S.close()


@pytest.mark.parametrize("period,use_graph", [(2, -1), (5, -1), (32, -1), (32, 0), (48, -1)])
def test_pmag_with_period_matches_oracle(period, use_graph, dev):
    """Periods below the 16-iteration window, a multiple of it (short windows, the rule
    only in the windows that end before a multiple of the period; captured and eager
    launches) and a longer non-multiple."""
    w = make_workload(2, "small")
    A = w.A
    lo, hi = 1e-4, 1e-2
    L = mpcg.cg_tilecsc_from_csr(A.n, A.indptr, A.indices, A.data, w.R, w.C)
    Lo = otc.build(A.n, A.indptr, A.indices, A.data, w.R, w.C)
    ref = ocg.solve(Lo, A.indptr, A.indices, A.data, w.b,
                    ocg.PMagSchedule(Lo.C, Lo.tile_col_idx, lo, hi, period), w.tol, 1000, keep_maps=False)
    S = mpcg.Solver(L, use_graph=use_graph)
    S.cg_set_schedule_pmag(lo, hi, period)
    bd = torch.from_numpy(w.b).to(dev)
    xd = torch.zeros_like(bd)
    status, K, hist = S.cg_solve(bd, xd, w.tol, 1000)
    log(f"pmag period {period} graph {use_graph}: GPU K={K}, oracle K={ref.K}")
    assert status == ref.status
    assert abs(K - ref.K) <= max(1, math.floor(0.02 * ref.K))
    ks, counts = S.cg_get_map_trace()
    assert ks.tolist() == list(range(0, K, period))
    for i, (k0, c, _) in enumerate(ref.windows):
        if k0 > min(K, ref.K) or abs(hist[k0] - ref.hist[k0]) > 1e-9 * ref.hist[k0]:
            break
        assert ks[i] == k0 and counts[i].tolist() == c, (i, k0)
    S.close()
