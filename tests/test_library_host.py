"""CPU tests of the C-ABI library: exported symbols, the host layout builder
(bit-exact against the oracle) and argument validation. No GPU calls."""

import ctypes as ct
import os
import re

import numpy as np
import pytest
import scipy.sparse as sp

from gen import make_workload
from oracle import tilecsc as otc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

mpcg = pytest.importorskip("mixed_precision_sparse_amd")
from mixed_precision_sparse_amd import _lib  # noqa: E402


def _declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"\b(cg_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))


def test_options_struct_matches_header():
    """The binding's cg_options has the header's fields, in order, with their sizes."""
    text = open(os.path.join(ROOT, "include", "mpcg.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    body = re.search(r"typedef struct \{(.*?)\} cg_options;", text, flags=re.S).group(1)
    fields = [(name, int(count) if count else 1) for name, count in re.findall(r"int32_t\s+(\w+)(?:\[(\d+)\])?;", body)]
    ours = [(name, ct.sizeof(typ) // 4) for name, typ in _lib.cg_options._fields_]
    assert fields == ours
    assert ct.sizeof(_lib.cg_options) == 4 * sum(c for _, c in fields)


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    names = _declared_functions()
    assert len(names) >= 20
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"
    assert lib.cg_version() >= 10000


def _compare_layout(L_lib, L_or):
    assert L_lib.T == L_or.T and L_lib.nnz == L_or.nnz
    assert np.array_equal(L_lib.tile_row_ptr, L_or.tile_row_ptr)
    assert np.array_equal(L_lib.tile_col_idx, L_or.tile_col_idx)
    assert np.array_equal(L_lib.tile_nnz_ptr, L_or.tile_nnz_ptr)
    assert np.array_equal(L_lib.row_idx, L_or.row_idx)
    assert np.array_equal(L_lib.col_local, L_or.col_local)
    assert np.array_equal(L_lib.perm(), L_or.perm)
    assert np.array_equal(L_lib.val, L_or.val)
    assert np.array_equal(L_lib.col_ptr(), L_or.col_ptr)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_host_layout_matches_oracle_on_workloads(cfg):
    w = make_workload(cfg, "small")
    A = w.A
    L_lib = mpcg.cg_tilecsc_from_csr(A.n, A.indptr, A.indices, A.data, w.R, w.C)
    L_or = otc.build(A.n, A.indptr, A.indices, A.data, w.R, w.C)
    _compare_layout(L_lib, L_or)


@pytest.mark.parametrize("R,C", [(1, 1), (3, 5), (16, 16), (32, 32), (64, 16), (256, 256), (100, 7),
                                 (257, 8), (300, 16), (512, 64), (4096, 32), (16384, 256)])
def test_host_layout_matches_oracle_random(R, C):
    n = 517
    M = sp.random(n, n, density=0.01, random_state=np.random.RandomState(R * 1000 + C), format="csr")
    M = (M + sp.eye(n, format="csr")).tolil()
    M[100:140, :] = 0  # empty rows
    M = M.tocsr()
    M.eliminate_zeros()
    M.data[::7] = 0.0  # explicit zeros stay structural
    M.sort_indices()
    L_lib = mpcg.cg_tilecsc_from_csr(n, M.indptr, M.indices, M.data, R, C)
    L_or = otc.build(n, M.indptr, M.indices, M.data, R, C)
    _compare_layout(L_lib, L_or)


def test_host_layout_empty_matrix():
    n = 10
    L = mpcg.cg_tilecsc_from_csr(n, np.zeros(n + 1, np.int64), np.zeros(0, np.int32),
                                 np.zeros(0), 4, 4)
    assert L.T == 0 and L.nnz == 0
    assert L.tile_row_ptr.tolist() == [0, 0, 0, 0]
    # The layout is valid, but no handle is made for it: a matrix without
    # nonzeros is not SPD. The check precedes every device call.
    lib = _lib.load()
    out = ct.c_void_p()
    assert lib.cg_create(L._h, None, None, None, ct.byref(out)) == mpcg.CG_EINVAL
    assert b"no nonzeros" in lib.cg_last_error() and not out.value


@pytest.mark.parametrize("case", ["unsorted", "duplicate", "out_of_range", "nan", "bad_R", "bad_R_tall",
                                  "bad_C", "n0", "rowptr"])
def test_host_layout_rejects_bad_input(case):
    n = 4
    indptr = np.array([0, 2, 3, 4, 5], np.int64)
    indices = np.array([0, 1, 1, 2, 3], np.int32)
    data = np.ones(5)
    R = C = 2
    if case == "unsorted":
        indices[:2] = [1, 0]
    elif case == "duplicate":
        indices[:2] = [1, 1]
    elif case == "out_of_range":
        indices[4] = 4
    elif case == "nan":
        data[2] = np.nan
    elif case == "bad_R":
        R = 0
    elif case == "bad_R_tall":
        R = 16385
    elif case == "bad_C":
        C = 257
    elif case == "n0":
        n = 0
    elif case == "rowptr":
        indptr[2] = 1
    with pytest.raises(mpcg.CGError) as ei:
        mpcg.cg_tilecsc_from_csr(n, indptr, indices, data, R, C)
    assert ei.value.code == mpcg.CG_EINVAL
    assert "cg_tilecsc_from_csr" in str(ei.value)


def test_null_arguments_return_einval_without_gpu():
    lib = _lib.load()
    assert lib.cg_tilecsc_from_csr(4, None, None, None, 2, 2, None) == mpcg.CG_EINVAL
    assert lib.cg_spmv(None, None, None, None) == mpcg.CG_EINVAL
    assert lib.cg_solve(None, None, None, 1e-8, 10, None, None, None, None) == mpcg.CG_EINVAL
    assert b"NULL" in lib.cg_last_error()
    assert lib.cg_destroy(None) == mpcg.CG_OK


def test_select_reuse_interval_matches_oracle():
    """The library's K* selection (host code) against the oracle on random records."""
    from oracle import maps as omaps

    rng = np.random.default_rng(3)
    for nrec, ncb in ((1, 5), (2, 3), (37, 11), (130, 64)):
        codes = (np.cumsum(rng.integers(-1, 2, (nrec, ncb)), axis=0) % 3).astype(np.uint8)
        for thr in (0.1, 0.3):
            k_ref, table_ref = omaps.select_reuse_interval(codes, thr)
            k, table = mpcg.cg_select_reuse_interval(codes, thr)
            assert k == k_ref
            assert [i for i, _ in table] == [i for i, _ in table_ref]
            assert np.allclose([f for _, f in table], [f for _, f in table_ref], rtol=0, atol=1e-15)


def test_select_reuse_interval_rejects_bad_codes():
    with pytest.raises(mpcg.CGError):
        mpcg.cg_select_reuse_interval(np.full((4, 2), 3, np.uint8))


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_tune_row_height_matches_oracle(cfg):
    """The library's row-block height search (host code) against the oracle: the chosen R and
    every count exactly (both sides compare candidates by the exact squared coefficient of
    variation); the reported coefficient and max/mean are two roundings of the same exact
    values, so they agree within a few units in the last place."""
    from gen import make_workload
    from oracle import tuning

    w = make_workload(cfg, "small")
    A = w.A
    for C, max_R, min_rb in ((64, 256, 1), (16, 16384, 4), (w.C, 256, 40)):
        R_ref, table_ref = tuning.tune_row_height(A.n, A.indptr, A.indices, C, max_R, min_rb)
        R, rows = mpcg.cg_tune_row_height(A.n, A.indptr, A.indices, C, max_R, min_rb)
        assert R == R_ref
        got = [(r["R"], r["row_blocks"], r["tiles"], r["admissible"]) for r in rows]
        assert got == [(t[0], t[1], t[2], t[5]) for t in table_ref]
        for r, t in zip(rows, table_ref):
            assert r["cv"] == pytest.approx(t[3], rel=4 * 2.0 ** -52, abs=0.0)
            assert r["max_ratio"] == pytest.approx(t[4], rel=4 * 2.0 ** -52, abs=0.0)


def test_tune_row_height_skewed_and_errors():
    from oracle import tuning

    rng = np.random.default_rng(5)
    n = 3000
    k = np.minimum((rng.pareto(1.1, n) + 1).astype(np.int64), n)
    indptr = np.concatenate([[0], np.cumsum(k)]).astype(np.int64)
    indices = np.concatenate([np.sort(rng.choice(n, kk, replace=False)) for kk in k]).astype(np.int32)
    for C in (1, 7, 64, 256):
        R_ref, table_ref = tuning.tune_row_height(n, indptr, indices, C, 16384, 2)
        R, rows = mpcg.cg_tune_row_height(n, indptr, indices, C, 16384, 2)
        assert R == R_ref
        assert [(r["R"], r["row_blocks"], r["tiles"], r["admissible"]) for r in rows] == \
            [(t[0], t[1], t[2], t[5]) for t in table_ref]
        for r, t in zip(rows, table_ref):
            assert r["cv"] == pytest.approx(t[3], rel=4 * 2.0 ** -52, abs=0.0)
            assert r["max_ratio"] == pytest.approx(t[4], rel=4 * 2.0 ** -52, abs=0.0)
    with pytest.raises(mpcg.CGError):
        mpcg.cg_tune_row_height(n, indptr, indices, 0)
    with pytest.raises(mpcg.CGError):
        mpcg.cg_tune_row_height(n, indptr, indices, 64, 256, 0)
    bad = indices.copy()
    bad[3] = n
    with pytest.raises(mpcg.CGError):
        mpcg.cg_tune_row_height(n, indptr, bad, 64)
