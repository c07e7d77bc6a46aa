"""GPU checks of the bandwidth references (measurement aids, no part of the method).

cg_stream_read must read every byte of its source once (its block sums add up
to the sum of the source), cg_stream_copy must copy exactly, and cg_stream_mix
must read as cg_stream_read does while writing every 16-byte pair of its
destination once. Sizes are small and ragged against the grid.
"""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
mpcg = pytest.importorskip("mixed_precision_sparse_amd")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    return torch.device("cuda:0")


def _src(dev, n, seed):
    return torch.from_numpy(np.random.default_rng(seed).uniform(-1, 1, n)).to(dev)


@pytest.mark.parametrize("n, blocks", [(2, 1), (2002, 3), (1 << 16, 64), (123458, 257)])
def test_stream_read_sums_every_entry(dev, n, blocks):
    src = _src(dev, n, n)
    sink = torch.full((blocks + 5,), float("nan"), dtype=torch.float64, device=dev)
    mpcg.cg_stream_read(src, sink, blocks)
    torch.cuda.synchronize()
    s = sink.cpu().numpy()
    assert np.isnan(s[blocks:]).all()  # nothing past the grid's blocks
    ref = float(np.sum(src.cpu().numpy()))
    assert abs(float(np.sum(s[:blocks])) - ref) <= 1e-12 * n


@pytest.mark.parametrize("n, blocks", [(2, 1), (2002, 3), (123458, 257)])
def test_stream_copy_is_exact(dev, n, blocks):
    src = _src(dev, n, n + 1)
    dst = torch.full_like(src, float("nan"))
    mpcg.cg_stream_copy(src, dst, blocks)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)


@pytest.mark.parametrize("n, m, blocks", [(2, 0, 1), (2002, 2, 3), (2002, 2002, 3), (123458, 9818, 257),
                                          (1 << 16, 4096, 64), (4096, 65536, 8)])
def test_stream_mix_reads_everything_and_writes_every_pair(dev, n, m, blocks):
    src = _src(dev, n, n + 2)
    before = src.clone()
    big = torch.full((m + 2,), float("nan"), dtype=torch.float64, device=dev)
    dst = big[:m]
    sink = torch.zeros(blocks, dtype=torch.float64, device=dev)
    mpcg.cg_stream_mix(src, dst, sink, blocks)
    torch.cuda.synchronize()
    assert torch.equal(src, before)
    ref = float(np.sum(before.cpu().numpy()))
    assert abs(float(sink.sum().item()) - ref) <= 1e-12 * n
    d = big.cpu().numpy()
    assert np.isfinite(d[:m]).all()          # every pair written (with a finite running sum)
    assert np.isnan(d[m:]).all()             # nothing past the destination
    if m:
        pairs = d[:m].reshape(-1, 2)
        assert np.array_equal(pairs[:, 0], pairs[:, 1])  # a pair holds one running sum twice


def test_stream_bindings_check_the_sink(dev):
    src = _src(dev, 64, 3)
    with pytest.raises(ValueError):
        mpcg.cg_stream_read(src, torch.zeros(2, dtype=torch.float64, device=dev), 3)
    with pytest.raises(ValueError):
        mpcg.cg_stream_mix(src, torch.zeros(2, dtype=torch.float64, device=dev),
                           torch.zeros(1, dtype=torch.float64, device=dev), 2)
