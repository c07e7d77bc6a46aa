"""Pins for the oracle's value streams (FP32 and BF16 round-to-nearest-even from FP64).

The expected results come from the formats' definitions, enumerated from bit
patterns, not from the routine under test.
"""

import numpy as np
import pytest

from oracle import rounding as rd


def _all_bf16_positive_finite():
    h = np.arange(0x0000, 0x7F80, dtype=np.uint32)  # +0 .. largest finite
    v = (h << 16).view(np.float32).astype(np.float64)
    return h, v


def test_bf16_exact_values_roundtrip():
    h, v = _all_bf16_positive_finite()
    assert np.array_equal(rd.to_bf16_value(v), v)
    assert np.array_equal(rd.bf16_bits(v), h.astype(np.uint16))
    assert np.array_equal(rd.bf16_bits(-v)[1:], (h[1:] | 0x8000).astype(np.uint16))


def test_bf16_midpoints_exhaustive():
    """Every gap between adjacent bf16 values: midpoint ties to even, +-1 FP64 ulp goes to the side."""
    h, v = _all_bf16_positive_finite()
    h_next = h + 1
    v_next = (h_next << 16).view(np.float32).astype(np.float64)
    # The gap above the largest finite value ends at 2^128 (rounds to infinity).
    top = h == 0x7F7F
    v_next[top] = 2.0 ** 128
    mid = v + (v_next - v) / 2.0  # exact: both ends have 8 significant bits
    below = np.nextafter(mid, -np.inf)
    above = np.nextafter(mid, np.inf)
    exp_up = np.where(top, np.inf, v_next)
    for sign in (1.0, -1.0):
        assert np.array_equal(rd.to_bf16_value(sign * below), sign * v)
        assert np.array_equal(rd.to_bf16_value(sign * above), sign * exp_up)
        tie = np.where((h & 1) == 0, v, exp_up)
        assert np.array_equal(rd.to_bf16_value(sign * mid), sign * tie)


def test_bf16_special_values():
    tiny = 2.0 ** -133  # smallest bf16 subnormal
    cases = [
        (0.0, 0.0), (-0.0, -0.0), (tiny, tiny), (tiny / 2, 0.0),
        (np.nextafter(tiny / 2, 1), tiny), (1e-300, 0.0), (-1e-300, -0.0),
        (np.inf, np.inf), (-np.inf, -np.inf), (1e300, np.inf), (-1e39, -np.inf),
        (1.0, 1.0), (1.0 + 2.0 ** -8, 1.0), (1.0 + 3 * 2.0 ** -8, 1.0 + 2 ** -6),
    ]
    for a, e in cases:
        got = rd.to_bf16_value(np.array([a]))[0]
        assert got == e and np.signbit(got) == np.signbit(e), (a, got, e)
    assert np.isnan(rd.to_bf16_value(np.array([np.nan]))[0])
    assert rd.bf16_bits(np.array([np.nan]))[0] == 0x7FC0


def test_bf16_matches_torch_on_fp32_exact_inputs():
    """On FP32-representable inputs there is no double rounding, so torch's RNE cast must agree."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    t = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(rd.bf16_bits(f.astype(np.float64)), t)


def test_bf16_direct_rounding_differs_from_double_rounding():
    """A value just above a bf16 midpoint that FP32 rounds onto the midpoint: direct RNE goes up."""
    mid = 1.0 + 2.0 ** -8  # halfway between 1 and 1 + 2^-7
    a = mid + 2.0 ** -40  # FP32 would round this to exactly the midpoint, then tie to 1.0
    assert np.float32(a) == np.float32(mid)
    assert rd.to_bf16_value(np.array([a]))[0] == 1.0 + 2.0 ** -7


def test_fp32_midpoints_sampled():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 0x7F7FFFFF, size=100_000, dtype=np.int64).astype(np.uint32)
    v = bits.view(np.float32).astype(np.float64)
    vn = (bits + 1).view(np.float32).astype(np.float64)
    mid = v + (vn - v) / 2.0
    assert np.array_equal(rd.to_fp32(np.nextafter(mid, -np.inf)).astype(np.float64), v)
    assert np.array_equal(rd.to_fp32(np.nextafter(mid, np.inf)).astype(np.float64), vn)
    tie = np.where((bits & 1) == 0, v, vn)
    assert np.array_equal(rd.to_fp32(mid).astype(np.float64), tie)
    fmax = float(np.finfo(np.float32).max)
    half_ulp = 2.0 ** (127 - 24)
    assert rd.to_fp32(np.array([fmax + half_ulp]))[0] == np.inf
    assert rd.to_fp32(np.array([np.nextafter(fmax + half_ulp, 0)]))[0] == np.float32(fmax)
    sub = 2.0 ** -149
    assert rd.to_fp32(np.array([sub * 1.5]))[0] == np.float32(2 * sub)  # tie to even
    assert rd.to_fp32(np.array([sub * 0.5]))[0] == 0.0


def test_stream_values_selects_per_entry():
    a = np.array([1.0 + 2.0 ** -30, 1.0 + 2.0 ** -30, 1.0 + 2.0 ** -30, 3.0])
    out = rd.stream_values(a, np.array([0, 1, 2, 2]))
    assert out[0] == a[0]
    assert out[1] == 1.0 and out[2] == 1.0 and out[3] == 3.0
