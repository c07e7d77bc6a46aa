"""The C ABI from plain C: tests/c_abi_host.c is compiled as C99 against
include/mpcg.h, linked with the built library, and run (host calls only, no
GPU). Its output is compared with a layout derived by hand for a 5 x 5
tridiagonal matrix in 2 x 2 tiles (Sec. 3.3, Fig. 4: tiles row block by row
block, CSC inside a tile) and with the CPU oracle."""

import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import maps as omaps, tilecsc as otc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "mixed_precision_sparse_amd")


@pytest.fixture(scope="module")
def output(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    if not os.path.exists(os.path.join(LIB_DIR, "libmpcg.so")):
        pytest.skip("libmpcg.so not built")
    exe = str(tmp_path_factory.mktemp("cabi") / "c_abi_host")
    rocm_lib = "/opt/rocm/lib"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_abi_host.c"), "-o", exe, "-L", LIB_DIR, "-lmpcg",
           f"-Wl,-rpath,{LIB_DIR}", f"-Wl,-rpath-link,{rocm_lib}", f"-Wl,-rpath,{rocm_lib}"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    out = {}
    for line in run.stdout.splitlines():
        key, _, rest = line.partition(" ")
        out[key] = rest
    return out


def _ints(s):
    return [int(t) for t in s.split()]


# Hand derivation: rows {0,1}, {2,3}, {4} and the same column blocks. Row block 0
# touches column blocks 0 (4 entries) and 1 (entry (1,2)); row block 1 touches 0
# ((2,1)), 1 (4 entries) and 2 ((3,4)); row block 2 touches 1 ((4,3)) and 2 ((4,4)).
# Inside a tile the entries go column by column, rows ascending.
HAND = {
    "sizes": [5, 7, 13, 2, 2],
    "tile_row_ptr": [0, 2, 5, 7],
    "tile_col_idx": [0, 1, 0, 1, 2, 1, 2],
    "tile_nnz_ptr": [0, 4, 5, 6, 10, 11, 12, 13],
    "row_idx": [0, 1, 0, 1, 1, 0, 0, 1, 0, 1, 1, 0, 0],
    "col_local": [0, 0, 1, 1, 0, 1, 0, 0, 1, 1, 0, 1, 0],
    "val": [2, -1, -1, 2, -1, -1, 2, -1, -1, 2, -1, -1, 2],
}


def test_c_layout_matches_hand_derivation(output):
    assert _ints(output["sizes"]) == HAND["sizes"]
    for key in ("tile_row_ptr", "tile_col_idx", "tile_nnz_ptr", "row_idx", "col_local"):
        assert _ints(output[key]) == HAND[key], key
    assert [float(t) for t in output["val"].split()] == HAND["val"]


def test_c_layout_matches_oracle(output):
    rowptr = np.array([0, 2, 5, 8, 11, 13])
    colind = np.array([0, 1, 0, 1, 2, 1, 2, 3, 2, 3, 4, 3, 4])
    val = np.array([2, -1, -1, 2, -1, -1, 2, -1, -1, 2, -1, -1, 2], dtype=np.float64)
    Lo = otc.build(5, rowptr, colind, val, 2, 2)
    assert _ints(output["tile_row_ptr"]) == Lo.tile_row_ptr.tolist()
    assert _ints(output["tile_col_idx"]) == Lo.tile_col_idx.tolist()
    assert _ints(output["tile_nnz_ptr"]) == Lo.tile_nnz_ptr.tolist()
    assert _ints(output["row_idx"]) == Lo.row_idx.tolist()
    assert _ints(output["col_local"]) == Lo.col_local.tolist()
    assert _ints(output["col_ptr"]) == Lo.col_ptr.reshape(-1).tolist()
    # perm maps canonical order to CSR positions: the values agree through it
    perm = np.array(_ints(output["perm"]))
    assert np.array_equal(val[perm], Lo.val)
    assert sorted(perm.tolist()) == list(range(13))


def test_c_error_path_and_host_helpers(output):
    rc, nulled = _ints(output["unsorted_rc"])
    assert rc < 0 and nulled == 1
    assert "cg_tilecsc_from_csr" in output["unsorted_msg"]
    assert _ints(output["tune"]) == [10, 32]
    parts = output["reuse"].split()
    nk, kstar = int(parts[0]), int(parts[1])
    got = {int(p.split(":")[0]): float(p.split(":")[1]) for p in parts[2:]}
    codes = np.array([2, 1, 0, 1, 0, 1, 0, 1], dtype=np.uint8).reshape(4, 2)
    ref_kstar, ref = omaps.select_reuse_interval(codes, 0.1)
    assert kstar == ref_kstar == 1
    assert nk == len(ref) and got == {int(K): float(f) for K, f in ref}
    assert got == {1: 0.0, 2: 1.0}
    assert int(output["version"]) >= 10300
    # every stream reference rejects its bad arguments with CG_EINVAL (-1), no device call made
    assert _ints(output["stream_rc"]) == [-1] * 5
