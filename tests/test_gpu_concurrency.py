"""Handles are independent: two handles solving at the same time from two host
threads give the same bits as each solving alone, and errors are reported per
thread (cg_last_error is thread-local). ctypes releases the GIL during the
library calls, so the two solves overlap on the host and on the device."""

import sys
import threading

import numpy as np
import pytest

from gen import make_workload, static_map, tile_scores

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


def _handles(dev):
    """A static-map solve (3D Laplacian) and a Jacobi ratchet solve (power-law matrix), both
    multi-launch, plus one single-workgroup solve (2D Laplacian)."""
    out = []
    for cfg, sb in ((2, -1), (4, -1), (1, 1)):
        w = make_workload(cfg, "small")
        A = w.A
        L = mpcg.cg_tilecsc_from_csr(A.n, A.indptr, A.indices, A.data, w.R, w.C)
        S = mpcg.Solver(L, jacobi=w.jacobi, single_block=sb)
        if w.map_spec["kind"] == "static":
            S.cg_set_precision_map(static_map(tile_scores(L.T, 2)))
        elif w.map_spec["kind"] == "ratchet":
            S.cg_set_schedule_residual(w.map_spec["thresholds"], w.map_spec["prec"])
        b = torch.from_numpy(w.b).to(dev)
        out.append((f"cfg{cfg}", S, b, w))
    return out


def _solve(S, b, w, stream):
    x = torch.zeros_like(b)
    with torch.cuda.stream(stream):
        st, K, hist = S.cg_solve(b, x, w.tol, w.maxit, stream=stream)
    stream.synchronize()
    return st, K, hist, x.cpu().numpy()


def test_concurrent_solves_match_sequential(dev):
    hs = _handles(dev)
    streams = [torch.cuda.Stream() for _ in hs]
    torch.cuda.synchronize()
    ref = [_solve(S, b, w, s) for (_, S, b, w), s in zip(hs, streams)]
    for rep in range(3):
        got = [None] * len(hs)
        errors = []

        def run(i):
            try:
                _, S, b, w = hs[i]
                got[i] = _solve(S, b, w, streams[i])
            except Exception as e:  # reported below, on the main thread
                errors.append((i, repr(e)))

        threads = [threading.Thread(target=run, args=(i,)) for i in range(len(hs))]
        for t in threads:
            t.start()
        for t in threads:
            t.join(timeout=120)
        assert not any(t.is_alive() for t in threads), "a solve did not return"
        assert not errors, errors
        for (name, _, _, _), r, g in zip(hs, ref, got):
            assert (r[0], r[1]) == (g[0], g[1]), (name, rep, r[:2], g[:2])
            assert np.array_equal(r[2], g[2]) and np.array_equal(r[3], g[3]), (name, rep)
        log(f"round {rep}: " + ", ".join(f"{n} {g[0]} K={g[1]}" for (n, _, _, _), g in zip(hs, got)))
    for _, S, _, _ in hs:
        S.close()


def test_errors_are_reported_per_thread(dev):
    w = make_workload(2, "small")
    A = w.A
    L = mpcg.cg_tilecsc_from_csr(A.n, A.indptr, A.indices, A.data, w.R, w.C)
    S = mpcg.Solver(L)
    lib = mpcg._lib.load()
    seen = {}
    barrier = threading.Barrier(2)

    def failing():
        rc = lib.cg_set_schedule_pmag(S._h, 1.0, 0.5, 1)  # lo > hi: CG_EINVAL
        barrier.wait()
        barrier.wait()
        seen["failing"] = (rc, lib.cg_last_error().decode())

    def clean():
        barrier.wait()
        rc = lib.cg_set_precision_map(S._h, mpcg._ptr(np.zeros(L.T, np.uint8)), 0)
        seen["clean"] = (rc, lib.cg_last_error().decode())
        barrier.wait()

    t1, t2 = threading.Thread(target=failing), threading.Thread(target=clean)
    t1.start()
    t2.start()
    t1.join(timeout=60)
    t2.join(timeout=60)
    assert seen["failing"][0] < 0 and "cg_set_schedule_pmag" in seen["failing"][1]
    assert seen["clean"] == (0, "")
    S.close()
