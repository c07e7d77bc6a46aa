"""Pins for the per-segment max|p| rule (EvoCG paper, Sec. 4.7) and its schedule.

The rule is checked against a pure-Python loop over tiles and column entries
written straight from the definition, and at its threshold boundaries; the
schedule inside CG is checked against the two cases where it must reduce to
another, independently pinned oracle path: thresholds that no |p| can fall
below give the all-FP64 static run bit for bit, thresholds that every |p|
falls below give the all-BF16 static run bit for bit. A CG trace hook then
confirms, iteration by iteration, that the map in force is the rule applied
to the direction that iteration multiplies.
"""

import numpy as np
import pytest
import scipy.sparse as sp

from gen import make_workload
from oracle import cg, maps, spmv, tilecsc as tc


def _brute_force(p, C, tcol, lo, hi):
    out = []
    for J in tcol:
        m = 0.0
        for j in range(int(J) * C, min((int(J) + 1) * C, len(p))):
            m = max(m, abs(float(p[j])))
        out.append(2 if m < lo else (1 if m < hi else 0))
    return out


@pytest.mark.parametrize("n,C,seed", [(100, 16, 1), (37, 4, 2), (64, 32, 3), (5, 8, 4)])
def test_pmag_rule_matches_brute_force(n, C, seed):
    rng = np.random.default_rng(seed)
    p = rng.standard_normal(n) * 10.0 ** rng.uniform(-6, 0, n)
    tcol = rng.integers(0, -(-n // C), 200)
    for lo, hi in ((1e-4, 1e-3), (1e-3, 1e-1), (0.0, 0.5), (2.0, 3.0)):
        assert maps.pmag_rule(p, C, tcol, lo, hi).tolist() == _brute_force(p, C, tcol, lo, hi)


def test_pmag_rule_threshold_boundaries():
    """m = lo is FP32 (BF16 needs m < lo); m = hi is FP64 (FP32 needs m < hi)."""
    C = 4
    p = np.array([1e-3, -2e-4, 0.0, 0.0,   # block 0: m = 1e-3 = lo
                  0.0, 0.0, -1e-2, 0.0,    # block 1: m = 1e-2 = hi
                  0.0, 0.0, 0.0, 0.0,      # block 2: m = 0
                  5e-3])                   # block 3 (ragged): m = 5e-3
    got = maps.pmag_rule(p, C, np.array([0, 1, 2, 3, 1, 0]), 1e-3, 1e-2)
    assert got.tolist() == [1, 0, 2, 1, 0, 1]


def _cfg_small(cfg):
    w = make_workload(cfg, "small")
    A = w.A
    L = tc.build(A.n, A.indptr, A.indices, A.data, w.R, w.C)
    return w, A, L


@pytest.mark.parametrize("cfg", [2, 3])
def test_pmag_schedule_reduces_to_static_fp64_and_bf16(cfg):
    w, A, L = _cfg_small(cfg)
    for lo, hi, code in ((0.0, 0.0, 0), (np.inf, np.inf, 2)):
        rp = cg.solve(L, A.indptr, A.indices, A.data, w.b, cg.PMagSchedule(L.C, L.tile_col_idx, lo, hi),
                      w.tol, 300, keep_maps=False)
        rs = cg.solve(L, A.indptr, A.indices, A.data, w.b, cg.StaticSchedule(np.full(L.T, code, np.uint8)),
                      w.tol, 300, keep_maps=False)
        assert (rp.K, rp.status) == (rs.K, rs.status)
        assert rp.hist == rs.hist
        assert np.array_equal(rp.x, rs.x)


def test_pmag_schedule_applies_the_rule_to_each_direction():
    """Each iteration's product equals the SpMV under the rule's map for that p."""
    w, A, L = _cfg_small(2)
    lo, hi = 1e-4, 1e-2
    seen = []

    def hook(k, x, r, p, q, alpha):
        m = maps.pmag_rule(p, L.C, L.tile_col_idx, lo, hi)
        assert np.array_equal(q, spmv.spmv(L, A.indptr, A.indices, m, p))
        seen.append(np.bincount(m, minlength=3))

    res = cg.solve(L, A.indptr, A.indices, A.data, w.b, cg.PMagSchedule(L.C, L.tile_col_idx, lo, hi),
                   w.tol, 400, trace=hook, keep_maps=False)
    assert res.status == "converged"
    seen = np.array(seen)
    # As p shrinks the rule moves tiles down: the run visits all three precisions.
    assert seen[0, 0] == L.T and seen[:, 1].max() > 0 and seen[:, 2].max() > 0
    assert len(res.windows) == res.K and [c for _, c, _ in res.windows] == seen.tolist()


def test_pmag_spec_builds_the_schedule():
    w, A, L = _cfg_small(3)
    s = cg.schedule_for({"kind": "pmag", "lo": 1e-9, "hi": 1e-8}, L)
    p = np.linspace(-1, 1, A.n)
    assert np.array_equal(s.map_for(0, 1.0, L.T, p), maps.pmag_rule(p, L.C, L.tile_col_idx, 1e-9, 1e-8))
