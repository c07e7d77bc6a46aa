"""Pins for the oracle's mixed-precision SpMV and its map rules.

The SpMV is checked against a dense product whose entries are looked up tile
by tile from the definition (row // R, col // C) and rounded with NumPy's
float32 cast and torch's bfloat16 cast on inputs where those casts are
single roundings; the map rules against brute-force loops.
"""

import numpy as np
import pytest
import scipy.sparse as sp

from gen import make_workload
from oracle import maps, spmv, tilecsc as tc
from oracle.rounding import to_bf16_value


def _fp32_exact_matrix(n, density, seed):
    """Nonsymmetric sparse matrix whose values are FP32-exact with 16 significant bits."""
    rng = np.random.default_rng(seed)
    M = sp.random(n, n, density=density, random_state=np.random.RandomState(seed), format="csr")
    M = (M + sp.eye(n, format="csr")).tocsr()
    M.sort_indices()
    mant = rng.integers(2 ** 15, 2 ** 16, M.nnz)
    expo = rng.integers(-20, 20, M.nnz)
    sign = rng.choice([-1.0, 1.0], M.nnz)
    M.data = sign * np.ldexp(mant.astype(np.float64), expo - 16)
    return M


def _dense_reference(M, R, C, L, prec_of_tile):
    torch = pytest.importorskip("torch")
    tile_lookup = {}
    rb = L.tile_row_block()
    for t in range(L.T):
        tile_lookup[(int(rb[t]), int(L.tile_col_idx[t]))] = int(prec_of_tile[t])
    D = np.zeros(M.shape)
    coo = M.tocoo()
    for i, j, v in zip(coo.row, coo.col, coo.data):
        p = tile_lookup[(i // R, j // C)]
        if p == 0:
            D[i, j] = v
        elif p == 1:
            D[i, j] = float(np.float32(v))
        else:
            D[i, j] = float(torch.tensor(np.float32(v)).to(torch.bfloat16).float().item())
    return D


@pytest.mark.parametrize("n,R,C,seed", [(45, 8, 8, 1), (64, 16, 16, 2), (70, 16, 8, 3)])
def test_spmv_mixed_matches_dense_tile_lookup(n, R, C, seed):
    M = _fp32_exact_matrix(n, 0.1, seed)
    L = tc.build(n, M.indptr, M.indices, M.data, R, C)
    prec = np.random.default_rng(seed + 100).integers(0, 3, L.T).astype(np.uint8)
    x = np.random.default_rng(seed + 200).uniform(-1, 1, n)
    D = _dense_reference(M, R, C, L, prec)
    y_ref = D @ x
    bound = 1e-13 * (np.abs(D) @ np.abs(x))
    for y in (spmv.spmv(L, M.indptr, M.indices, prec, x),
              spmv.spmv_loop(L, M.indptr, M.indices, prec, x)):
        assert np.all(np.abs(y - y_ref) <= bound)


def test_spmv_fp64_map_matches_dense():
    M = _fp32_exact_matrix(80, 0.08, 9)
    M.data = M.data * (1.0 + 2.0 ** -40)  # not FP32-exact any more
    L = tc.build(80, M.indptr, M.indices, M.data, 16, 16)
    x = np.random.default_rng(3).uniform(-1, 1, 80)
    y = spmv.spmv(L, M.indptr, M.indices, np.zeros(L.T, np.uint8), x)
    y_ref = M.toarray() @ x
    assert np.all(np.abs(y - y_ref) <= 1e-13 * (np.abs(M.toarray()) @ np.abs(x)))


def test_spmv_wrong_tile_assignment_is_caught():
    """A transposed tile lookup (the map of tile (J, I) used for (I, J)) must change the result."""
    n, R, C = 64, 16, 16
    M = _fp32_exact_matrix(n, 0.2, 4)
    M.data = M.data * (1.0 + 2.0 ** -20)
    L = tc.build(n, M.indptr, M.indices, M.data, R, C)
    prec = np.random.default_rng(5).integers(0, 3, L.T).astype(np.uint8)
    x = np.ones(n)
    good = spmv.spmv(L, M.indptr, M.indices, prec, x)
    MT = M.T.tocsr()
    MT.sort_indices()
    LT = tc.build(n, MT.indptr, MT.indices, MT.data, R, C)
    assert LT.T == L.T
    # Same map applied to the transposed structure gives different rounding somewhere.
    bad = spmv.spmv(LT, MT.indptr, MT.indices, prec, x)
    assert not np.allclose(good, bad, rtol=1e-12, atol=0)


@pytest.mark.parametrize("cfg", [1, 2])
def test_integer_stencils_are_exact_in_every_precision(cfg):
    """Values 4, 6, -1 are exact in BF16 and FP32, so every map gives the FP64 result bit for bit."""
    w = make_workload(cfg, "small")
    A = w.A
    L = tc.build(A.n, A.indptr, A.indices, A.data, w.R, w.C)
    x = np.random.default_rng(1).uniform(-1, 1, A.n)
    y64 = spmv.spmv(L, A.indptr, A.indices, np.zeros(L.T, np.uint8), x)
    for p in (1, 2):
        assert np.array_equal(spmv.spmv(L, A.indptr, A.indices, np.full(L.T, p, np.uint8), x), y64)
    mixed = np.random.default_rng(2).integers(0, 3, L.T).astype(np.uint8)
    assert np.array_equal(spmv.spmv(L, A.indptr, A.indices, mixed, x), y64)


def test_magnitude_rule_brute_force():
    w = make_workload(3, "small")
    A = w.A
    L = tc.build(A.n, A.indptr, A.indices, A.data, 16, 16)
    got = maps.magnitude_rule(L, 1e-4, 1e-2)
    S = A.to_scipy()
    dmax = np.abs(S.diagonal()).max()
    rb = L.tile_row_block()
    expect = []
    for t in range(L.T):
        I, J = int(rb[t]), int(L.tile_col_idx[t])
        blk = S[I * 16:(I + 1) * 16, J * 16:(J + 1) * 16]
        ratio = np.abs(blk.data).max() / dmax
        expect.append(2 if ratio < 1e-4 else (1 if ratio < 1e-2 else 0))
    assert got.tolist() == expect
    assert set(np.unique(got)) == {0, 1, 2}  # the small cfg3 exercises all three classes


def test_ratchet_thresholds_inclusive_and_one_way():
    r = maps.Ratchet((1e-3, 1e-6), (2, 1, 0))
    seq = [1.0, 0.5, 1e-3, 5e-3, 2e-4, 1e-6, 1.0]
    assert [r.step(s) for s in seq] == [2, 2, 1, 1, 1, 0, 0]
    r2 = maps.Ratchet((1e-3, 1e-6), (2, 1, 0))
    assert r2.step(1e-7) == 0  # both thresholds passed at once


def test_tile_rule_brute_force():
    s = np.random.default_rng(2).random(1000)
    for rho in (1.0, 3e-3, 1e-4, 2e-6, 1e-9):
        got = maps.tile_rule(s, rho, 1e-3, 1e-6)
        exp = [2 if v * rho > 1e-3 else (1 if v * rho > 1e-6 else 0) for v in s]
        assert got.tolist() == exp


def test_bf16_stream_used_for_bf16_tiles():
    """One tile, all three codes: the product uses exactly the rounded value."""
    a = 1.0 + 2.0 ** -10 + 2.0 ** -30
    M = sp.csr_matrix(np.array([[a]]))
    L = tc.build(1, M.indptr, M.indices, M.data, 1, 1)
    x = np.array([3.0])
    assert spmv.spmv(L, M.indptr, M.indices, np.array([0], np.uint8), x)[0] == a * 3.0
    assert spmv.spmv(L, M.indptr, M.indices, np.array([1], np.uint8), x)[0] == \
        float(np.float32(a)) * 3.0
    assert spmv.spmv(L, M.indptr, M.indices, np.array([2], np.uint8), x)[0] == \
        float(to_bf16_value(np.array([a]))[0]) * 3.0


def test_spmv_rows_matches_full_product():
    M = _fp32_exact_matrix(90, 0.1, 12)
    M.data = M.data * (1.0 + 2.0 ** -30)
    R = C = 16
    L = tc.build(90, M.indptr, M.indices, M.data, R, C)
    prec = np.random.default_rng(13).integers(0, 3, L.T).astype(np.uint8)
    x = np.random.default_rng(14).uniform(-1, 1, 90)
    y = spmv.spmv(L, M.indptr, M.indices, prec, x)
    keys, _ = tc.tile_numbering(90, M.indptr, M.indices, R, C)
    rows = [0, 5, 17, 44, 89]
    yr = spmv.spmv_rows(M.indptr, M.indices, M.data, rows,
                        lambda i, cols: prec[tc.tile_of(keys, 90, R, C, np.full(cols.size, i), cols)], x)
    assert np.allclose(yr, y[rows], rtol=1e-15, atol=0)


@pytest.mark.parametrize("n,R,C,seed", [(45, 8, 8, 1), (70, 16, 8, 3), (97, 32, 16, 5)])
def test_spmv_full_matches_dense_tile_lookup_and_spmv(n, R, C, seed):
    """The full-size form (tiles from sorted keys, no Tile-CSC object) against the dense
    tile-by-tile reference, and bit for bit against spmv (same CSR order, same rounding)."""
    M = _fp32_exact_matrix(n, 0.1, seed)
    M.data = M.data * (1.0 + 2.0 ** -30)  # values no longer FP32-exact: the rounding matters
    L = tc.build(n, M.indptr, M.indices, M.data, R, C)
    prec = np.random.default_rng(seed + 100).integers(0, 3, L.T).astype(np.uint8)
    x = np.random.default_rng(seed + 200).uniform(-1, 1, n)
    y = spmv.spmv_full(n, M.indptr, M.indices, M.data, R, C, prec, x)
    assert np.array_equal(y, spmv.spmv(L, M.indptr, M.indices, prec, x))
    M2 = _fp32_exact_matrix(n, 0.1, seed)
    L2 = tc.build(n, M2.indptr, M2.indices, M2.data, R, C)
    D = _dense_reference(M2, R, C, L2, prec)
    y2 = spmv.spmv_full(n, M2.indptr, M2.indices, M2.data, R, C, prec, x)
    assert np.all(np.abs(y2 - D @ x) <= 1e-13 * (np.abs(D) @ np.abs(x)))
    # the tile of every entry matters: a map shifted by one tile changes the product
    y3 = spmv.spmv_full(n, M.indptr, M.indices, M.data, R, C, np.roll(prec, 1), x)
    assert not np.array_equal(y3, y)
