"""Pins of the oracle's 1x128 / 128x128 quantisers: properties fixed by the
scale rule (every nonzero tile reaches 448), the E4M3 error bound, power-of-two
scale invariance, tile independence, and a brute-force scalar loop."""
import math

import numpy as np

from oracle import formats as F
from oracle import quant as Q


def _rand_tiles(M, K, seed):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((M, K)).astype(np.float32)
    v *= np.exp(rng.uniform(-6, 6, (M, 1))).astype(np.float32)  # per-row dynamic range
    return v


def test_every_nonzero_tile_reaches_448():
    v = _rand_tiles(64, 1024, 1)
    q, s = Q.quant_1x128(v)
    mags = np.abs(F.e4m3_decode(q)).reshape(64, 8, 128).max(axis=2)
    assert np.all(mags == 448.0)
    assert s.shape == (64, 8) and s.dtype == np.float32


def test_error_bound_half_ulp():
    v = _rand_tiles(32, 512, 2)
    q, s = Q.quant_1x128(v)
    deq = Q.dequant_1x128(q, s)
    scaled = (v.reshape(32, 4, 128) / s[:, :, None]).reshape(32, 512).astype(np.float64)
    a = np.abs(scaled)
    # ulp of E4M3 at |x|: 2^(floor(log2|x|) - 3), 2^-9 in the subnormal range
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    ulp = 2.0 ** (e - 3)
    err = np.abs(deq - v.astype(np.float64)) / np.repeat(s, 128, axis=1)
    assert np.all(err <= 0.5 * ulp + 1e-12)


def test_zero_tile_scale_one_and_sign():
    v = np.zeros((2, 256), np.float32)
    v[1, :128] = -0.0
    v[1, 128] = 3.0
    q, s = Q.quant_1x128(v)
    assert s[0, 0] == 1.0 and s[0, 1] == 1.0 and s[1, 0] == 1.0
    assert np.all(q[0] == 0)
    assert np.all(q[1, :128] == 0x80)          # -0 keeps its sign
    assert q[1, 128] == 0x7E and s[1, 1] == np.float32(3.0) / np.float32(448.0)


def test_power_of_two_invariance():
    v = _rand_tiles(16, 384, 3)
    q1, s1 = Q.quant_1x128(v)
    q2, s2 = Q.quant_1x128(v * np.float32(2.0 ** 5))
    assert np.array_equal(q1, q2)
    assert np.array_equal(s2, s1 * np.float32(32.0))


def test_tiles_are_independent():
    v = _rand_tiles(4, 512, 4)
    q1, s1 = Q.quant_1x128(v)
    v2 = v.copy()
    v2[2, 130] = 1e4                             # row 2, tile 1 only
    q2, s2 = Q.quant_1x128(v2)
    changed = np.argwhere(s1 != s2)
    assert changed.tolist() == [[2, 1]]
    diff = np.argwhere(q1 != q2)
    assert np.all(diff[:, 0] == 2) and np.all((diff[:, 1] >= 128) & (diff[:, 1] < 256))


def test_brute_force_scalar_loop():
    # One row quantised with a plain scalar loop from the rule's words:
    # scale = fp32(amax / 448); code = nearest E4M3 of fp32(v / scale).
    v = _rand_tiles(1, 256, 5)[0]
    q, s = Q.quant_1x128(v[None, :])
    for t in range(2):
        tile = v[t * 128:(t + 1) * 128]
        amax = max(abs(float(a)) for a in tile)
        scale = np.float32(np.float32(amax) / np.float32(448.0))
        assert s[0, t] == scale
        for j, a in enumerate(tile):
            x = float(np.float32(a) / scale)
            best = None
            for c in range(256):
                if c in (0x7F, 0xFF):
                    continue
                val = F.e4m3_value(c)
                if math.copysign(1.0, val) != math.copysign(1.0, x):
                    continue
                d = abs(val - min(max(x, -448.0), 448.0))
                if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
                    best = (d, c)
            assert q[0, t * 128 + j] == best[1]


def test_block_128x128():
    rng = np.random.default_rng(6)
    w = (rng.standard_normal((256, 384)) * 0.02).astype(np.float32)
    w[128:, 256:] *= 100                         # one block with a wider range
    q, s = Q.quant_128x128(w)
    assert s.shape == (2, 3)
    blocks = np.abs(F.e4m3_decode(q)).reshape(2, 128, 3, 128).max(axis=(1, 3))
    assert np.all(blocks == 448.0)
    for i in range(2):
        for j in range(3):
            blk = w[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            assert s[i, j] == np.float32(np.abs(blk).max()) / np.float32(448.0)
    # a 128x128 block quantised alone equals its part of the matrix
    qb, sb = Q.quant_128x128(w[128:, 256:])
    assert np.array_equal(qb, q[128:, 256:]) and sb[0, 0] == s[1, 2]
    deq = Q.dequant_128x128(q, s)
    assert np.max(np.abs(deq - w) / np.repeat(np.repeat(s, 128, 0), 128, 1)) <= 16.0 + 1e-9
