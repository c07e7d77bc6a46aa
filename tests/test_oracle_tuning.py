"""Pins for the row-block height tuning of the oracle (EvoCG, Sec. 3.3.3).

Tile counts per row block against brute-force sets of (row block, column
block) pairs and against the pinned layout builder; the balance measure in
closed form on an identity matrix; the selection rule (smallest coefficient
of variation, admissibility by height and row-block count, ties to the
smaller R) on hand-built cases.
"""

import math

import numpy as np
import pytest
import scipy.sparse as sp

from oracle import tilecsc as tc, tuning


def _random_csr(n, density, seed):
    M = sp.random(n, n, density=density, random_state=np.random.RandomState(seed), format="csr")
    M = (M + sp.eye(n, format="csr")).tocsr()
    M.sort_indices()
    return M


@pytest.mark.parametrize("n,R,C,seed", [(50, 3, 5, 1), (97, 8, 8, 2), (200, 32, 7, 3), (64, 64, 64, 4)])
def test_tile_counts_match_brute_force_sets(n, R, C, seed):
    M = _random_csr(n, 0.05, seed)
    counts = tuning.row_block_tile_counts(n, M.indptr, M.indices, R, C)
    per_block = [set() for _ in range(-(-n // R))]
    coo = M.tocoo()
    for i, j in zip(coo.row, coo.col):
        per_block[i // R].add(j // C)
    assert counts.tolist() == [len(s) for s in per_block]
    L = tc.build(n, M.indptr, M.indices, M.data, R, C)
    assert counts.sum() == L.T
    assert np.array_equal(counts, np.diff(L.tile_row_ptr))


def test_balance_closed_form_on_identity():
    # identity, n = 1000, R = 32, C = 8: 31 full row blocks with 4 diagonal tiles, the last (8 rows) with 1
    n = 1000
    I = sp.eye(n, format="csr")
    counts = tuning.row_block_tile_counts(n, I.indptr, I.indices, 32, 8)
    assert counts.tolist() == [4] * 31 + [1]
    mean = (31 * 4 + 1) / 32
    var = (31 * (4 - mean) ** 2 + (1 - mean) ** 2) / 32
    cv, mx = tuning.balance(counts)
    assert cv == pytest.approx(math.sqrt(var) / mean, rel=1e-14)
    assert mx == pytest.approx(4 / mean, rel=1e-14)
    assert tuning.balance(np.zeros(5)) == (0.0, 0.0)
    assert tuning.balance(np.full(7, 3)) == (0.0, 1.0)


def _arrow(n, heavy_row):
    """Diagonal plus one dense row: only the heavy row's block has extra tiles."""
    rows = list(range(n)) + [heavy_row] * n
    cols = list(range(n)) + list(range(n))
    M = sp.csr_matrix((np.ones(len(rows)), (rows, cols)), shape=(n, n))
    M.sum_duplicates()
    M.sort_indices()
    return M


def test_selection_rule_hand_cases():
    n = 256
    M = _arrow(n, 0)
    cands = (4, 8, 16, 32)
    # by hand (C = 4, ncb = 64): R = 4 -> 64 blocks, block 0 has 64 tiles, the others 1;
    # R = 8 -> 32 blocks, block 0 has 64, the others 2; R = 16 -> 16 blocks, 64 vs 4;
    # R = 32 -> 8 blocks, 64 vs 8. The coefficient of variation falls as R grows.
    R, table = tuning.tune_row_height(n, M.indptr, M.indices, 4, max_R=32, min_row_blocks=1, candidates=cands)
    cvs = [row[3] for row in table]
    assert [row[2] for row in table] == [64 + 63, 64 + 31 * 2, 64 + 15 * 4, 64 + 7 * 8]
    assert cvs == sorted(cvs, reverse=True)
    assert R == 32
    # the height limit and the row-block floor exclude candidates
    assert tuning.tune_row_height(n, M.indptr, M.indices, 4, max_R=16, min_row_blocks=1, candidates=cands)[0] == 16
    assert tuning.tune_row_height(n, M.indptr, M.indices, 4, max_R=32, min_row_blocks=16, candidates=cands)[0] == 16
    assert tuning.tune_row_height(n, M.indptr, M.indices, 4, max_R=32, min_row_blocks=17, candidates=cands)[0] == 8
    # nothing admissible: the smallest candidate
    assert tuning.tune_row_height(n, M.indptr, M.indices, 4, max_R=2, min_row_blocks=1, candidates=cands)[0] == 4
    # admissibility is recorded per row
    _, t2 = tuning.tune_row_height(n, M.indptr, M.indices, 4, max_R=16, min_row_blocks=32, candidates=cands)
    assert [row[5] for row in t2] == [True, True, False, False]


def test_selection_ties_go_to_the_smaller_height():
    # identity with C = 4: every row block of R >= 4 rows holds R / 4 tiles, so every cv is 0
    n = 512
    I = sp.eye(n, format="csr")
    R, table = tuning.tune_row_height(n, I.indptr, I.indices, 4, max_R=64, min_row_blocks=1,
                                      candidates=(8, 16, 32, 64))
    assert all(row[3] == 0.0 for row in table)
    assert R == 8


def test_default_candidates_are_the_papers_powers_of_two():
    assert tuning.CANDIDATES == (32, 64, 128, 256, 512, 1024, 2048, 4096, 8192, 16384)


def _skewed(n, seed):
    """Rows of power-law length at uniform columns (a small stand-in for the power-law workload)."""
    rng = np.random.default_rng(seed)
    k = np.minimum((rng.pareto(1.2, n) + 1).astype(np.int64), n // 2)
    rows = np.repeat(np.arange(n), k)
    cols = rng.integers(0, n, rows.size)
    M = sp.csr_matrix((np.ones(rows.size), (rows, cols)), shape=(n, n)) + sp.eye(n, format="csr")
    M = M.tocsr()
    M.sum_duplicates()
    M.sort_indices()
    return M


def test_selection_minimises_cv_not_max_ratio():
    """The tuned R is the admissible row with the smallest cv; on these inputs the smallest
    max/mean would pick differently at least once."""
    cands = (4, 8, 16, 32, 64)
    disagree = 0
    for seed in range(12):
        M = _skewed(600, seed)
        R, table = tuning.tune_row_height(600, M.indptr, M.indices, 8, max_R=64, min_row_blocks=8,
                                          candidates=cands)
        adm = [row for row in table if row[5]]
        best = min(adm, key=lambda row: (row[3], row[0]))
        assert R == best[0]
        disagree += min(adm, key=lambda row: (row[4], row[0]))[0] != R
    assert disagree > 0


def test_cv_squared_exact_against_the_definition():
    """cv^2 in rational arithmetic equals the textbook population variance over the squared
    mean written element by element, and matches FP64 NumPy where NumPy is accurate."""
    from fractions import Fraction

    rng = np.random.default_rng(3)
    for _ in range(20):
        c = rng.integers(0, 50, rng.integers(1, 40))
        if c.sum() == 0:
            continue
        m = len(c)
        mean = Fraction(int(c.sum()), m)
        var = sum((Fraction(int(v)) - mean) ** 2 for v in c) / m
        assert tuning.cv_squared(c) == var / mean ** 2
        assert math.sqrt(float(tuning.cv_squared(c))) == pytest.approx(float(np.std(c) / np.mean(c)), rel=1e-12)
    assert tuning.cv_squared(np.zeros(4, dtype=np.int64)) == 0
    assert tuning.cv_squared(np.array([5, 5, 5])) == 0


def test_selection_orders_a_near_tie_exactly():
    """A hand-built near tie: counts (p, p+1) against (q, q, q, q, q+1) with 5q = 4p + 2.
    Exactly cv_a^2 = 1/(2p+1)^2 and cv_b^2 = 4/(4p+3)^2, so b is smaller, by a relative
    1/(4p) ~ 2.5e-18: below FP64 resolution, where the usual formulas tie (and so would
    pick the smaller height, a). The selection must still take b."""
    from fractions import Fraction

    p = 10 ** 17 + 2
    q = (4 * p + 2) // 5
    assert 5 * q == 4 * p + 2
    a = np.array([p, p + 1], dtype=np.int64)
    b = np.array([q, q, q, q, q + 1], dtype=np.int64)
    assert tuning.cv_squared(a) == Fraction(1, (2 * p + 1) ** 2)
    assert tuning.cv_squared(b) == Fraction(4, (4 * p + 3) ** 2)
    # FP64 cannot tell them apart: the rounded measures and NumPy's std/mean agree bit for bit
    def fp64_cv(c):  # sqrt(m S2 - S1^2) / S1 with the exact integers rounded once each
        c = [int(v) for v in c]
        m, s1, s2 = len(c), sum(c), sum(v * v for v in c)
        return math.sqrt(float(m * s2 - s1 * s1)) / float(s1)

    assert fp64_cv(a) == fp64_cv(b)
    assert float(np.std(a.astype(np.float64)) / np.mean(a.astype(np.float64))) == \
        float(np.std(b.astype(np.float64)) / np.mean(b.astype(np.float64)))
    assert tuning.balance(a)[0] == tuning.balance(b)[0]
    # the exact comparison orders them, whichever comes first
    assert tuning.select_height([(32, a), (64, b)], max_R=64, min_row_blocks=1) == 64
    assert tuning.select_height([(32, b), (64, a)], max_R=64, min_row_blocks=1) == 32
    # equal exact values keep the smaller height
    assert tuning.select_height([(32, a), (64, a.copy())], max_R=64, min_row_blocks=1) == 32
