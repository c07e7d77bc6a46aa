"""GPU test of cg_true_residual_noalloc, the entry point for callers that cannot
allocate: its value against cg_true_residual's (same kernels: bit for bit) and
against the oracle's FP64 residual, on two calls in a row, the second on a
smaller system (fewer partial sums than the first left in the static scratch).
"""

import numpy as np
import pytest

from gen import make_workload
from oracle import spmv as ospmv

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
mpcg = pytest.importorskip("mixed_precision_sparse_amd")


def test_noalloc_true_residual_matches_allocating_call():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    out = torch.full((1,), float("nan"), dtype=torch.float64, device=dev)
    for cfg, seed in ((2, 3), (1, 4)):  # the second system is smaller
        w = make_workload(cfg, "small")
        A = w.A
        print(f"noalloc residual cfg{cfg} n={A.n}", flush=True)
        L = mpcg.cg_tilecsc_from_csr(A.n, A.indptr, A.indices, A.data, w.R, w.C)
        S = mpcg.Solver(L, single_block=-1)
        x = np.random.default_rng(seed).uniform(-1, 1, A.n)
        bd = torch.from_numpy(w.b).to(dev)
        xd = torch.from_numpy(x).to(dev)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        S.cg_true_residual_noalloc(bd, xd, out)
        torch.cuda.synchronize()
        got = float(out.cpu()[0])
        want = S.cg_true_residual(bd, xd)
        assert got == want
        ref = float(np.linalg.norm(w.b - A.to_scipy() @ x) / np.linalg.norm(w.b))
        s = ospmv.abs_bound(A.indptr, A.indices, A.data, x) + np.abs(w.b)
        assert abs(got - ref) <= 2.5e-13 * float(np.linalg.norm(s)) / float(np.linalg.norm(w.b))
        S.close()
