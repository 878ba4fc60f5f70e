"""Number formats, written from their definitions (test infrastructure only).

E4M3FN (OCP 8-bit floating point, E4M3 variant): 1 sign bit, 4 exponent bits
with bias 7, 3 mantissa bits.  Exponent field 0 holds subnormals
(m/8 * 2^-6); fields 1..15 hold (1 + m/8) * 2^(e-7); S.1111.111 is NaN;
there is no infinity.  Largest finite value 448, smallest subnormal 2^-9.

The pages only say "FP8" (news.qq.com/rain/a/20241229A05OQF00, section
FP8 低精度训练; aliyun study note section 4.1).  The reading used here:
E4M3FN, round to nearest with ties to even, saturate to +-448 (no NaN from
overflow), and keep the sign of zero.

bf16: 1 sign, 8 exponent (bias 127), 7 mantissa bits; rounding to nearest
with ties to even.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_NAN_CODES = (0x7F, 0xFF)


def e4m3_value(code: int) -> float:
    """Value of one E4M3FN code, straight from the bit fields."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** (1 - 7)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# decode table for all 256 codes (float64, NaN at 0x7F / 0xFF)
E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
# magnitudes of the non-negative finite codes 0x00..0x7E, ascending
_MAGS = E4M3_TABLE[:0x7F].copy()


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Encode real values (float32/float64) to E4M3FN codes.

    Nearest representable magnitude, ties to the even code (even mantissa),
    magnitudes >= 448 saturate to 448, sign bit copied (so -0 -> 0x80).
    NaN input is not defined for this path and is mapped to 0x7F.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    sign = np.signbit(v).astype(np.uint8) << 7
    # lo = largest code whose magnitude <= a
    lo = np.searchsorted(_MAGS, a, side="right") - 1
    lo = np.clip(lo, 0, 0x7E)
    hi = np.minimum(lo + 1, 0x7E)
    mlo = _MAGS[lo]
    mhi = _MAGS[hi]
    mid = 0.5 * (mlo + mhi)  # exact in float64
    pick_hi = (a > mid) | ((a == mid) & (lo % 2 == 1))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    out = (code.astype(np.uint8) | sign).astype(np.uint8)
    out = np.where(np.isnan(v), np.uint8(0x7F), out).astype(np.uint8)
    return out


def bf16_round(v: np.ndarray) -> np.ndarray:
    """Round real values to the nearest bf16 value (ties to even), as float64.

    One rounding from the exact value: quantum 2^(e-7) in binade
    [2^e, 2^(e+1)), 2^-133 below the normal range.  np.rint is round half to
    even, and v / quantum is exact (power-of-two scaling).
    """
    v = np.asarray(v, dtype=np.float64)
    _, ex = np.frexp(v)          # v = m * 2^ex, m in [0.5, 1)
    e = np.maximum(ex - 1, -126)
    quantum = np.ldexp(1.0, e - 7)
    r = np.rint(v / quantum) * quantum
    r = np.where(np.abs(r) > 3.3895313892515355e38, np.copysign(np.inf, v), r)
    return np.where(v == 0, v, r)


def bf16_bits_from_value(v: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of values that are already bf16-representable."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def bf16_value_from_bits(b: np.ndarray) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
