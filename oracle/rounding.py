"""Value streams: FP64 kept, FP32 and BF16 by one round-to-nearest-even step from FP64.

The paper keeps three pre-quantised value streams per nonzero and selects
one per tile (EvoCG, Sec. 3.3.2 "Intra-Tile CSC Execution"; Sec. 4.8
"Memory cost"). It does not state the rounding; this oracle takes IEEE
round-to-nearest-even, applied once to the FP64 value (no detour through
FP32 for BF16), subnormals kept, overflow to infinity.

Test infrastructure only: see the package docstring.
"""

from __future__ import annotations

import numpy as np

# Largest finite bfloat16: (2 - 2^-7) * 2^127.
BF16_MAX = float.fromhex("0x1.fep127")


def to_fp32(a: np.ndarray) -> np.ndarray:
    """FP32 stream: the IEEE RNE conversion of each FP64 value (overflow goes to infinity)."""
    with np.errstate(over="ignore"):
        return np.asarray(a, dtype=np.float64).astype(np.float32)


def to_bf16_value(a: np.ndarray) -> np.ndarray:
    """BF16 stream as FP64 numbers (exact): RNE of ``a`` to 8 significant bits.

    Written from the format's definition: a value a = m * 2^e with
    0.5 <= |m| < 1 is a normal bfloat16 multiple of 2^(e-8); below 2^-126
    the spacing is fixed at 2^-133 (subnormals). Scaling by a power of two is
    exact in FP64, and ``np.rint`` rounds half to even, so
    rint(a / q) * q is the correctly rounded result for spacing q.
    """
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)
    q_exp = np.maximum(e.astype(np.int64) - 8, -133)
    with np.errstate(invalid="ignore", over="ignore"):
        y = np.rint(np.ldexp(a, -q_exp))
        r = np.ldexp(y, q_exp)
        r = np.where(np.isfinite(a) & (np.abs(r) > BF16_MAX), np.copysign(np.inf, a), r)
    return r


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """BF16 stream as uint16 bit patterns (NaN maps to the canonical quiet NaN 0x7FC0)."""
    v = to_bf16_value(a).astype(np.float32)  # exact: v has <= 8 significant bits
    bits = (v.view(np.uint32) >> 16).astype(np.uint16)
    nan = np.isnan(v)
    if nan.any():
        bits = bits.copy()
        bits[nan] = 0x7FC0
    return bits


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to FP64 (exact)."""
    u32 = np.asarray(bits, dtype=np.uint32) << 16
    return u32.view(np.float32).astype(np.float64)


def stream_values(a: np.ndarray, prec: np.ndarray) -> np.ndarray:
    """Per-entry stored value widened back to FP64: prec 0 -> a, 1 -> fp32(a), 2 -> bf16(a)."""
    a = np.asarray(a, dtype=np.float64)
    prec = np.asarray(prec)
    out = a.copy()
    m32 = prec == 1
    if m32.any():
        out[m32] = to_fp32(a[m32]).astype(np.float64)
    m16 = prec == 2
    if m16.any():
        out[m16] = to_bf16_value(a[m16])
    return out
