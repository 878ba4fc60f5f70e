"""Pins of the oracle's number formats against the format definitions,
hand-derived golden points and torch's independent CPU casts."""
import os

import numpy as np
import pytest
import torch

from conftest import GOLDEN
from oracle import formats as F


def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            rows.append((float(parts[0]), int(parts[1], 16)))
    return rows


def test_e4m3_table_shape():
    t = F.E4M3_TABLE
    finite = np.isfinite(t)
    assert finite.sum() == 254
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x01] == 2.0 ** -9
    assert t[0x08] == 2.0 ** -6
    assert t[0x38] == 1.0
    # magnitudes strictly increase over 0x00..0x7E and mirror for negatives
    assert np.all(np.diff(t[:0x7F]) > 0)
    assert np.array_equal(t[0x80:0xFF], -t[0x00:0x7F])
    assert np.signbit(t[0x80]) and t[0x80] == 0


def test_e4m3_table_matches_torch_decode():
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn)
    td = codes.to(torch.float64).numpy()
    mine = F.E4M3_TABLE
    both_nan = np.isnan(td) & np.isnan(mine)
    assert np.all(both_nan | (td == mine))
    assert np.array_equal(np.signbit(td[~both_nan]), np.signbit(mine[~both_nan]))


def test_e4m3_roundtrip_every_code():
    codes = np.array([c for c in range(256) if c not in F.E4M3_NAN_CODES], dtype=np.uint8)
    assert np.array_equal(F.e4m3_encode(F.e4m3_decode(codes)), codes)


def test_e4m3_golden_points():
    rows = _golden("e4m3_points.txt")
    vals = np.array([r[0] for r in rows])
    exp = np.array([r[1] for r in rows], dtype=np.uint8)
    got = F.e4m3_encode(vals)
    assert np.array_equal(got, exp), list(zip(vals, got, exp))


def test_e4m3_midpoints_go_to_even():
    mags = F.E4M3_TABLE[:0x7F]
    for c in range(0x7E):
        mid = 0.5 * (mags[c] + mags[c + 1])
        even = c if c % 2 == 0 else c + 1
        assert F.e4m3_encode(np.array([mid]))[0] == even
        assert F.e4m3_encode(np.array([-mid]))[0] == (even | 0x80)
        assert F.e4m3_encode(np.array([np.nextafter(mid, 0)]))[0] == c
        assert F.e4m3_encode(np.array([np.nextafter(mid, 1e9)]))[0] == c + 1


def test_e4m3_matches_torch_cast_in_range():
    # torch's CPU cast rounds to nearest even but does not saturate, so
    # compare only where |x| < 464 (the midpoint to the NaN pattern).
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * 100,
        rng.standard_normal(100000).astype(np.float32) * 0.01,
        rng.standard_normal(50000).astype(np.float32) * 1e-3,
        rng.uniform(-463.9, 463.9, 50000).astype(np.float32),
    ])
    x = x[np.abs(x) < 464]
    tq = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.e4m3_encode(x), tq)


def test_e4m3_saturates():
    big = np.array([448.0, 448.00003, 463.99, 464.0, 1e4, 1e30, -449.0, -1e30])
    assert np.array_equal(F.e4m3_encode(big), np.array([0x7E] * 6 + [0xFE] * 2, np.uint8))


def test_bf16_golden_points():
    for v, bits in _golden("bf16_points.txt"):
        r = F.bf16_round(np.array([v]))
        assert F.bf16_bits_from_value(r)[0] == bits, (v, hex(F.bf16_bits_from_value(r)[0]))


def test_bf16_matches_torch_on_fp32():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(300000) * s for s in (1e-30, 1e-3, 1.0, 1e3, 1e30)])
    x32 = x.astype(np.float32)
    tb = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    mine = F.bf16_round(x32.astype(np.float64))
    assert np.array_equal(tb, mine)


def test_bf16_single_rounding_from_float64():
    # a float64 value just above a bf16 midpoint whose float32 rounding would
    # land exactly on the midpoint: one rounding must go up, not to even.
    mid = 1.0 + 2.0 ** -8           # midpoint between 1 and 1 + 2^-7
    v = mid + 2.0 ** -40             # not representable in float32
    assert np.float32(v) == np.float32(mid)
    assert F.bf16_round(np.array([v]))[0] == 1.0 + 2.0 ** -7
    assert F.bf16_round(np.array([mid]))[0] == 1.0


def test_bf16_value_bits_roundtrip():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    v = F.bf16_value_from_bits(bits)
    ok = np.isfinite(v)
    assert np.array_equal(F.bf16_bits_from_value(v[ok]), bits[ok])
    assert np.array_equal(F.bf16_round(v[ok]), v[ok])
