"""Pins for the oracle's canonical Tile-CSC layout.

Checked against: a brute-force construction straight from the definition
(pure Python over a dict of entries), SciPy's CSC of every tile block, the
round trip back to CSR, and the worked example printed in the paper's
Fig. 4(a)/(b) (fixtures under tests/golden/).
"""

import json
import os

import numpy as np
import pytest
import scipy.sparse as sp

from oracle import tilecsc as tc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def random_csr(n, density, seed, empty_rows=(), explicit_zero=True, nonsym=True):
    rng = np.random.default_rng(seed)
    M = sp.random(n, n, density=density, random_state=np.random.RandomState(seed), format="csr")
    M = M + sp.eye(n, format="csr")
    M = M.tolil()
    for i in empty_rows:
        M[i, :] = 0
    M = M.tocsr()
    M.eliminate_zeros()
    if explicit_zero and M.nnz:
        M.data[rng.integers(0, M.nnz)] = 0.0  # structural entry with value 0
    M.sort_indices()
    return M


def brute_force(n, indptr, indices, data, R, C):
    entries = {}
    for i in range(n):
        for k in range(indptr[i], indptr[i + 1]):
            entries[(i, int(indices[k]))] = (k, float(data[k]))
    nrb = -(-n // R)
    ncb = -(-n // C)
    trp, tci, tnp, cps, ri, perm = [0], [], [0], [], [], []
    for I in range(nrb):
        cnt = 0
        for J in range(ncb):
            cols = []
            for c in range(C):
                col = [r for r in range(R) if (I * R + r, J * C + c) in entries]
                cols.append(col)
            nnz_t = sum(len(col) for col in cols)
            if nnz_t == 0:
                continue
            cnt += 1
            tci.append(J)
            cp = [0]
            for c, col in enumerate(cols):
                for r in col:
                    ri.append(r)
                    perm.append(entries[(I * R + r, J * C + c)][0])
                cp.append(cp[-1] + len(col))
            cps.append(cp)
            tnp.append(tnp[-1] + nnz_t)
        trp.append(trp[-1] + cnt)
    return trp, tci, tnp, cps, ri, perm


CASES = [
    # n, density, seed, R, C, empty rows
    (37, 0.08, 1, 4, 4, (3, 4, 5, 6, 7)),      # an empty row block, ragged tail
    (50, 0.05, 2, 16, 16, ()),                 # ragged in both directions
    (33, 0.2, 3, 8, 16, (0,)),                 # non-square tiles
    (20, 0.3, 4, 1, 1, ()),                    # 1x1 tiles
    (70, 0.02, 5, 32, 8, (60, 61, 62, 63, 64, 65, 66, 67, 68, 69)),  # empty last row block
    # Row blocks taller than 256 rows (Sec. 3.3.3 tunes R up to 16384): row
    # offsets past one byte, a height that is not a power of two, one row
    # block taller than the matrix.
    (611, 0.01, 6, 300, 16, tuple(range(250, 290))),
    (700, 0.006, 7, 512, 64, ()),
    (530, 0.008, 8, 16384, 32, ()),
]


@pytest.mark.parametrize("n,density,seed,R,C,empty", CASES)
def test_layout_matches_brute_force(n, density, seed, R, C, empty):
    M = random_csr(n, density, seed, empty)
    L = tc.build(n, M.indptr, M.indices, M.data, R, C)
    trp, tci, tnp, cps, ri, perm = brute_force(n, M.indptr, M.indices, M.data, R, C)
    assert L.tile_row_ptr.tolist() == trp
    assert L.tile_col_idx.tolist() == tci
    assert L.tile_nnz_ptr.tolist() == tnp
    assert L.col_ptr.tolist() == cps
    assert L.row_idx.tolist() == ri
    assert L.perm.tolist() == perm
    assert np.array_equal(L.val, M.data[L.perm])


@pytest.mark.parametrize("n,density,seed,R,C,empty", CASES)
def test_layout_matches_scipy_csc_per_tile(n, density, seed, R, C, empty):
    M = random_csr(n, density, seed, empty)
    L = tc.build(n, M.indptr, M.indices, M.data, R, C)
    rb = L.tile_row_block()
    for t in range(L.T):
        I, J = int(rb[t]), int(L.tile_col_idx[t])
        blk = M[I * R:(I + 1) * R, J * C:(J + 1) * C].tocsc()
        blk.sort_indices()
        s, e = int(L.tile_nnz_ptr[t]), int(L.tile_nnz_ptr[t + 1])
        cp = np.zeros(C + 1, dtype=np.int64)
        cp[:blk.indptr.size] = blk.indptr
        cp[blk.indptr.size:] = blk.indptr[-1]
        assert np.array_equal(L.col_ptr[t], cp)
        assert np.array_equal(L.row_idx[s:e], blk.indices)
        assert np.array_equal(L.val[s:e], blk.data)


@pytest.mark.parametrize("n,density,seed,R,C,empty", CASES)
def test_layout_round_trip_and_counts(n, density, seed, R, C, empty):
    M = random_csr(n, density, seed, empty)
    L = tc.build(n, M.indptr, M.indices, M.data, R, C)
    assert L.nnz == M.nnz
    assert int(np.diff(L.tile_nnz_ptr).sum()) == M.nnz
    assert np.all(np.diff(L.tile_nnz_ptr) > 0)  # only non-empty tiles are listed
    ip, ind, val = tc.to_csr(L)
    assert np.array_equal(ip, M.indptr)
    assert np.array_equal(ind, M.indices)
    assert np.array_equal(val, M.data)


def _last_block(n, C):
    return -(-n // C) - 1


def test_fig4a_inter_tile_csr():
    g = json.load(open(os.path.join(GOLDEN, "fig4a_inter_tile_csr.json")))
    n, R, C = g["n"], g["R"], g["C"]
    cols = [_last_block(n, C) if v == "N/C" else v for v in g["tileColIdx"]]
    rows, cidx = [], []
    ptr = g["tileRowPtr"]
    for I in range(len(ptr) - 1):
        for t in range(ptr[I], ptr[I + 1]):
            rows.append(I * R + 5)
            cidx.append(cols[t] * C + 7)
    M = sp.csr_matrix((np.ones(len(rows)), (rows, cidx)), shape=(n, n))
    M.sort_indices()
    L = tc.build(n, M.indptr, M.indices, M.data, R, C)
    assert L.tile_row_ptr.tolist() == ptr
    assert L.tile_col_idx.tolist() == cols


def test_fig4b_intra_tile_csc_padded_view():
    g = json.load(open(os.path.join(GOLDEN, "fig4b_intra_tile_csc.json")))
    R, C = g["R"], g["C"]
    n = 2 * C
    rows, cols = [], []
    for c, rs in g["columns"].items():
        for r in rs:
            rows.append(r)
            cols.append(int(c))
    M = sp.csr_matrix((np.ones(len(rows)), (rows, cols)), shape=(n, n))
    M.sort_indices()
    L = tc.build(n, M.indptr, M.indices, M.data, R, C)
    ptr, ridx = tc.padded_columns(L, 0)
    assert ptr[:3] == g["padded_colPtr_head"]
    assert ptr[-1] == g["padded_colPtr_last"]
    for c, expect in g["padded_rowIdx"].items():
        exp = [R - 1 if v == "R-1" else (R if v == "R" else v) for v in expect]
        assert ridx[int(c)] == exp


@pytest.mark.parametrize("n,density,seed,R,C,empty", CASES)
def test_tile_numbering_matches_layout(n, density, seed, R, C, empty):
    M = random_csr(n, density, seed, empty)
    L = tc.build(n, M.indptr, M.indices, M.data, R, C)
    keys, trp = tc.tile_numbering(n, M.indptr, M.indices, R, C)
    assert np.array_equal(trp, L.tile_row_ptr)
    coo = M.tocoo()
    t = tc.tile_of(keys, n, R, C, coo.row, coo.col)
    # Canonical tile of each CSR entry from the full layout.
    t_full = np.empty(M.nnz, dtype=np.int64)
    t_full[L.perm] = L.tile_of_nnz()
    assert np.array_equal(t, t_full)
