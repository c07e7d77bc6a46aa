"""Full-size GPU parity: the five workloads at their real sizes.

Expected values come from the oracle: the layout digests, map digests and
CG results in tests/golden/cg_cfg*_full.json (written by
tests/golden/make_golden.py, which calls only gen and oracle), and the SpMV
compared on every row with the oracle's product of the rounded matrix
(oracle.spmv.spmv_full), under the FP64 map, a random mixed map and the
workload's own map (for the windowed tile rule: the map left by a short
solve whose later windows change it without a repack; the product reads
every tile from its precision's plane).
"""

import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import pytest

from gen import make_workload, static_map, tile_scores
from oracle import maps as omaps, spmv as ospmv, tilecsc as otc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
mpcg = pytest.importorskip("mixed_precision_sparse_amd")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def sha(a, dtype):
    return hashlib.sha256(np.ascontiguousarray(a, dtype=dtype).tobytes()).hexdigest()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    return torch.device("cuda:0")


_cache = {}


def workload(cfg):
    path = os.path.join(GOLDEN, f"cg_cfg{cfg}_full.json")
    if not os.path.exists(path):
        pytest.skip(f"no stored oracle results for cfg{cfg} (run tests/golden/make_golden.py {cfg})")
    if cfg not in _cache:
        _cache.clear()
        t = time.time()
        w = make_workload(cfg, "full")
        log(f"cfg{cfg}: generated n={w.n} nnz={w.A.nnz} in {time.time() - t:.1f}s")
        t = time.time()
        L = mpcg.cg_tilecsc_from_csr(w.A.n, w.A.indptr, w.A.indices, w.A.data, w.R, w.C)
        log(f"cfg{cfg}: Tile-CSC T={L.T} in {time.time() - t:.1f}s")
        _cache[cfg] = (w, L, json.load(open(path)))
    return _cache[cfg]


def true_residuals_agree(tr, tr_ref, tol, rel=1e-2):
    a, b = max(tr, tol), max(tr_ref, tol)
    return abs(a - b) <= rel * b


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_fullsize_layout_and_spmv(cfg, dev):
    w, L, g = workload(cfg)
    A = w.A
    assert w.input_hash() == g["input_hash"]
    assert (L.T, L.nnz) == (g["T"], g["nnz"])
    S = mpcg.Solver(L)
    e = S.cg_export_layout()
    for name, dtype in (("tile_row_ptr", np.int64), ("tile_col_idx", np.int32), ("tile_nnz_ptr", np.int64),
                        ("row_idx", np.uint8), ("col_local", np.uint8)):
        assert sha(e[name], dtype) == g["layout"][name], name
    del e
    log(f"cfg{cfg}: device layout digests equal the oracle's")

    # Every row at full size, in the launch configuration cg_spmv uses, against the
    # oracle's product of the rounded matrix (oracle.spmv.spmv_full).
    t = time.time()
    keys, _ = otc.tile_numbering(A.n, A.indptr, A.indices, w.R, w.C)
    log(f"cfg{cfg}: oracle tile numbering in {time.time() - t:.1f}s")
    rng = np.random.default_rng(100 + cfg)
    x = rng.uniform(-1, 1, A.n)
    xd = torch.from_numpy(x).to(dev)
    yd = torch.empty_like(xd)
    bound_all = 1e-13 * ospmv.abs_bound(A.indptr, A.indices, A.data, x)

    def check_all_rows(name, m):
        S.cg_spmv(xd, yd)
        torch.cuda.synchronize()
        y = yd.cpu().numpy()
        t0 = time.time()
        y_ref = ospmv.spmv_full(A.n, A.indptr, A.indices, A.data, w.R, w.C, m, x, keys=keys)
        bad = np.nonzero(~(np.abs(y - y_ref) <= bound_all))[0]
        assert bad.size == 0, (name, int(bad.size), bad[:5].tolist())
        log(f"cfg{cfg}: SpMV {name} map, all {A.n} rows within 1e-13*(|A||x|) (oracle {time.time() - t0:.1f}s)")

    for name, m in (("fp64", np.zeros(L.T, np.uint8)), ("random mixed", static_map(tile_scores(L.T, 7)))):
        S.cg_set_precision_map(m)
        check_all_rows(name, m)

    # The workload's own map at full size: the map itself against the oracle's rule, then
    # every row of the product under it.
    kind = w.map_spec["kind"]
    sc = tile_scores(L.T, 2)
    if kind == "static":
        m = static_map(sc, w.map_spec["frac_bf16"], w.map_spec["frac_fp32"])
        S.cg_set_precision_map(m)
        check_all_rows("own static", m)
    if kind == "magnitude":
        S.cg_map_from_magnitude(w.map_spec["t_bf16"], w.map_spec["t_fp32"])
        m = S.cg_get_active_map()
        assert sha(m, np.uint8) == g["runs"]["mixed"]["windows"][0]["sha"]
        log(f"cfg{cfg}: magnitude-rule map equals the oracle's")
        check_all_rows("magnitude rule", m)
    if kind == "ratchet":
        S.cg_set_schedule_residual(w.map_spec["thresholds"], w.map_spec["prec"])  # cg_spmv: the first stage
        check_all_rows("ratchet first stage", np.full(L.T, w.map_spec["prec"][0], np.uint8))
    if kind == "tile_rule":
        S.cg_set_schedule_tile_rule(10, sc, w.map_spec["hi"], w.map_spec["lo"])
        for rho in (1.0, 2.5e-3, 4e-6, 1e-9):
            S.cg_eval_tile_rule(rho)
            assert np.array_equal(S.cg_get_active_map(), omaps.tile_rule(sc, rho, w.map_spec["hi"], w.map_spec["lo"]))
        log(f"cfg{cfg}: tile-rule maps equal the oracle's")
        # A short solve: its windows at k = 10 and 20 change the map without any repack;
        # the product afterwards reads every tile from its precision's plane.
        bd = torch.from_numpy(w.b).to(dev)
        xs = torch.zeros_like(bd)
        st, K, hist = S.cg_solve(bd, xs, w.tol, 25)
        assert K == 25
        m = S.cg_get_active_map()
        assert np.array_equal(m, omaps.tile_rule(sc, hist[20], w.map_spec["hi"], w.map_spec["lo"]))
        check_all_rows("tile rule window k=20 (after in-solve map changes)", m)
    S.close()


def _configure(S, w, L):
    kind = w.map_spec["kind"]
    sc = tile_scores(L.T, 2)
    if kind == "static":
        S.cg_set_precision_map(static_map(sc, w.map_spec["frac_bf16"], w.map_spec["frac_fp32"]))
    elif kind == "magnitude":
        S.cg_map_from_magnitude(w.map_spec["t_bf16"], w.map_spec["t_fp32"])
    elif kind == "ratchet":
        S.cg_set_schedule_residual(w.map_spec["thresholds"], w.map_spec["prec"])
    elif kind == "tile_rule":
        S.cg_set_schedule_tile_rule(w.map_spec["period"], sc, w.map_spec["hi"], w.map_spec["lo"])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
@pytest.mark.parametrize("which", ["fp64", "mixed"])
def test_fullsize_cg(cfg, which, dev):
    w, L, g = workload(cfg)
    A = w.A
    ref = g["runs"][which]
    S = mpcg.Solver(L, jacobi=w.jacobi)
    if which == "mixed":
        _configure(S, w, L)
    bd = torch.from_numpy(w.b).to(dev)
    xd = torch.zeros_like(bd)
    t = time.time()
    status, K, hist = S.cg_solve(bd, xd, w.tol, w.maxit)
    el = time.time() - t
    x = xd.cpu().numpy()
    tr = float(np.linalg.norm(w.b - A.to_scipy() @ x) / np.linalg.norm(w.b))
    log(f"cfg{cfg} {which}: GPU K={K} {status} rho={hist[-1]:.3e} true={tr:.3e} ({el:.2f}s); "
        f"oracle K={ref['K']} {ref['status']} rho={ref['hist'][-1]:.3e} true={ref['true_residual']:.3e}")
    assert status == ref["status"]
    assert abs(K - ref["K"]) <= max(1, math.floor(0.02 * ref["K"]))
    assert true_residuals_agree(tr, ref["true_residual"], w.tol), (tr, ref["true_residual"])
    m = min(K, ref["K"], 20)
    assert np.allclose(hist[: m + 1], ref["hist"][: m + 1], rtol=1e-6, atol=0)
    ks, counts = S.cg_get_map_trace()
    wins = ref["windows"]
    if w.map_spec["kind"] in ("fp64", "static", "magnitude") or which == "fp64":
        assert ks.tolist() == [0] and counts[0].tolist() == wins[0]["counts"]
    elif w.map_spec["kind"] == "ratchet":
        assert ks.tolist() == [x["k"] for x in wins] and counts.tolist() == [x["counts"] for x in wins]
    else:
        agree = 0
        for i, win in enumerate(wins):
            k0 = win["k"]
            if i >= len(ks) or k0 > min(K, ref["K"]) or abs(hist[k0] - ref["hist"][k0]) > 1e-9 * ref["hist"][k0]:
                break
            assert ks[i] == k0 and counts[i].tolist() == win["counts"], (i, k0)
            agree += 1
        log(f"cfg{cfg} {which}: {agree} of {len(wins)} windows compared while trajectories agree")
        assert agree >= 1
    S.close()
