"""The quantisers' quotient x / s through the reciprocal (CPU, exact arithmetic).

The HIP quantisers compute the codes' quotient x / s as
    y = RN(1/s),  q = RN(x*y),  r = RN(x - q*s) (one FMA),  q' = RN(q + r*y) (one FMA)
with the sign of q restored on a zero result.  Markstein's theorem on division
through a correctly rounded reciprocal says q' = RN(x/s) for fp32 operands
whose residual does not underflow; the kernels take this path only for scales
in [2^-90, 2^100].  This checks the identity bit for bit (signed zeros
included) with exact rational arithmetic: bf16 inputs and their tile scales
amax/448, zeros of both signs, and divisors with extreme significands.  The
quantisers' GPU tests then compare the codes with the oracle's x / s.
"""
import math
import struct
from fractions import Fraction as F

import numpy as np


def _rn32(fr):
    """Round a nonzero rational to the nearest fp32 (ties to even)."""
    sgn = -1.0 if fr < 0 else 1.0
    fr = abs(fr)
    e = fr.numerator.bit_length() - fr.denominator.bit_length()
    while F(2) ** e > fr:
        e -= 1
    while F(2) ** (e + 1) <= fr:
        e += 1
    e = max(e, -126)
    m = fr / F(2) ** (e - 23)
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > F(1, 2) or (rem == F(1, 2) and fl % 2 == 1):
        fl += 1
    return sgn * float(fl * F(2) ** (e - 23))


def _mul(x, y):
    r = F(x) * F(y)
    return _rn32(r) if r else math.copysign(0.0, math.copysign(1.0, x) * math.copysign(1.0, y))


def _div(x, y):
    r = F(x) / F(y)
    return _rn32(r) if r else math.copysign(0.0, math.copysign(1.0, x) * math.copysign(1.0, y))


def _fma(x, y, z):
    prod = F(x) * F(y)
    tot = prod + F(z)
    if tot:
        return _rn32(tot)
    # exact zero: -0 only when both addends are zeros of negative sign
    psign = math.copysign(1.0, x) * math.copysign(1.0, y)
    neg = prod == 0 and F(z) == 0 and psign < 0 and math.copysign(1.0, z) < 0
    return -0.0 if neg else 0.0


def _bits(v):
    return struct.unpack("<I", struct.pack("<f", v))[0]


def _bf16(v):
    u = np.float32(v).view(np.uint32)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return float(np.uint32(u).view(np.float32))


def _recip_div(x, s):
    y = _div(1.0, s)
    q = _mul(x, y)
    r = _fma(-q, s, x)
    return math.copysign(_fma(r, y, q), q)


def test_reciprocal_division_equals_division_bitwise():
    rng = np.random.default_rng(7)
    n = 0
    for _ in range(1500):
        col = [_bf16(v) for v in rng.standard_normal(3) * 10.0 ** rng.uniform(-20, 20)]
        amax = max(abs(c) for c in col)
        if amax == 0:
            continue
        s = float(np.float32(amax) / np.float32(448.0))
        assert 2.0 ** -90 <= s <= 2.0 ** 100
        for x in col + [amax, -amax, 0.0, -0.0]:
            assert _bits(_recip_div(x, s)) == _bits(_div(x, s)), (x, s)
            n += 1
    assert n > 5000


def test_reciprocal_division_extreme_significands():
    rng = np.random.default_rng(8)
    for sig in (0xFFFFFF, 0xFFFFFE, 0x800001, 0x800000, 0xAAAAAB):
        for e in (-40, -3, 0, 30):
            s = float(np.float32(sig * 2.0 ** (e - 23)))
            for x in rng.standard_normal(150):
                x = _bf16(x * s * 300)
                assert _bits(_recip_div(x, s)) == _bits(_div(x, s)), (x, s)
