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

import math

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


# ---------------------------------------------------------------------------
# Interval reuse and the offline K* selection (Sec. 3.4).
# ---------------------------------------------------------------------------
def _delayed_fraction_loops(codes, interval):
    up = delayed = 0
    for k in range(1, len(codes)):
        s = (k // interval) * interval
        for J in range(len(codes[0])):
            if codes[k][J] < codes[k - 1][J]:
                up += 1
                if codes[s][J] > codes[k][J]:
                    delayed += 1
    return delayed / up if up else 0.0


def test_delayed_fraction_hand_cases():
    # One block climbing BF16 -> FP32 at k = 3 and FP32 -> FP64 at k = 6.
    c = np.array([[2], [2], [2], [1], [1], [1], [0], [0], [0], [0], [0], [0], [0], [0], [0], [0]], np.uint8)
    assert maps.delayed_upward_fraction(c, 1) == 0.0
    assert maps.delayed_upward_fraction(c, 2) == 0.5   # k = 3 waits for k = 4; k = 6 is a window start
    assert maps.delayed_upward_fraction(c, 4) == 1.0   # both wait
    assert maps.select_reuse_interval(c)[0] == 1
    # Transitions only at multiples of 8: reuse up to 8 delays nothing.
    c = np.full((24, 3), 2, np.uint8)
    c[8:, 0] = 1
    c[16:, 1] = 0
    # At 16 the rise at k = 8 waits for k = 16, the one at k = 16 starts a window.
    assert [f for _, f in maps.select_reuse_interval(c)[1]] == [0.0, 0.0, 0.0, 0.0, 0.5]
    assert maps.select_reuse_interval(c)[0] == 8
    # Only downward moves: nothing to delay, the largest candidate wins.
    c = np.array([[0, 0], [0, 1], [1, 1], [2, 2], [2, 2]], np.uint8)
    best, table = maps.select_reuse_interval(c)
    assert best == 4 and [i for i, _ in table] == [1, 2, 4]


def test_delayed_fraction_matches_loops():
    rng = np.random.default_rng(9)
    for trial in range(5):
        c = np.cumsum(rng.integers(-1, 2, (40, 7)), axis=0) % 3
        c = c.astype(np.uint8)
        for interval in (1, 2, 3, 4, 8, 16):
            assert math.isclose(maps.delayed_upward_fraction(c, interval),
                                _delayed_fraction_loops(c.tolist(), interval), rel_tol=0, abs_tol=0)


def test_select_threshold_is_strict():
    # Exactly 1 of 10 upward transitions delayed at interval 2: 0.1 is not below 0.1.
    c = np.full((21, 10), 2, np.uint8)
    for J in range(10):
        k = 2 * (J + 1) if J else 1  # block 0 rises at k = 1 (delayed at interval 2), the rest at even k
        c[k:, J] = 1
    assert maps.delayed_upward_fraction(c, 2) == 0.1
    assert maps.select_reuse_interval(c, 0.1)[0] == 1
    assert maps.select_reuse_interval(c, 0.11)[0] >= 2


def test_pmag_schedule_with_period_reuses_the_window_start_map():
    w, A, L = _cfg_small(2)
    lo, hi, period = 1e-4, 1e-2, 4
    recorded = []
    starts = {}

    def hook(k, x, r, p, q, alpha):
        if k % period == 0:
            starts[k] = p.copy()
        m = maps.pmag_rule(starts[(k // period) * period], L.C, L.tile_col_idx, lo, hi)
        assert np.array_equal(q, spmv.spmv(L, A.indptr, A.indices, m, p))

    res = cg.solve(L, A.indptr, A.indices, A.data, w.b,
                   cg.PMagSchedule(L.C, L.tile_col_idx, lo, hi, period, recorded), w.tol, 400, trace=hook,
                   keep_maps=False)
    assert res.status == "converged"
    assert [k for k, _, _ in res.windows] == list(range(0, res.K, period))
    assert len(recorded) == len(res.windows)
    for (k, _, _), codes in zip(res.windows, recorded):
        assert np.array_equal(codes, maps.pmag_column_codes(starts[k], L.C, lo, hi))
