"""Precision of gfx950's FP8 matrix instructions: the measured basis of the
MFMA term in the GEMM tolerances of the other tests, and of the exact-sum
form the small-group GEMM launches use.

FP32 accumulation of FP8 products is the pages' rule (news.qq.com/rain/a/
20241229A05OQF00, section FP8 低精度训练 › 提高累加精度, where the matrix
unit's own accumulation is too narrow and partial sums are promoted to FP32
at a fixed interval).  On gfx950 the FP8 instructions add the products of
each run of 8 consecutive K positions after truncating every product toward
zero to a multiple of 2^(e - 13), 2^e the binade of the run's largest
product; the runs' sums are added in FP32.  test_mfma_truncation_rule pins
that rule with hand-built dot products; test_mfma_error_within_rule checks
random dot products against the bound it implies; the empirical terms the
other tests use (2^-14 and 2^-12 of the sum of |products| per 128-term
block) are checked on the operand distributions those tests feed.

The vehicle is grouped_fp8_wgrad with one 128-token chunk per group and unit
scales: its FP32 output is one 128-term FP8 dot product per element (two
chained v_mfma_f32_32x32x64_f8f6f4 over tokens 0..63 and 64..127 of the
chunk) times 1.  The oracle's grouped_wgrad gives the exact sums (products of
E4M3 values and their 128-term sums are exact in float64).
"""
import numpy as np
import pytest
import torch

import fp8_block_scaled_bias_amd as M
from gpu_common import dev, host, log
from oracle import formats as OF
from oracle import gemm as OG
from oracle import quant as OQ

pytestmark = pytest.mark.gpu


def _wgrad_dots(y, a):
    """y, a: [G, 128 columns, 128 tokens] E4M3 codes -> GPU fp32 [G, 128, 128]
    (dot products of y's and a's columns over the chunk's tokens)."""
    G = y.shape[0]
    cap = 2 * G                      # the layout's capacity: ceil(M/128) + G chunks
    yc = np.zeros((cap, 128, 128), np.uint8)
    ac = np.zeros((cap, 128, 128), np.uint8)
    yc[:G], ac[:G] = y, a
    ones = np.ones((cap, 128), np.float32)
    offs = (np.arange(G + 1) * 128).astype(np.int32)
    dW = torch.empty((G, 128, 128), dtype=torch.float32, device="cuda")
    M.grouped_fp8_wgrad(dev(yc), dev(ones), dev(ac), dev(ones), cap, dev(offs), G, G * 128, 128,
                        128, dW)
    return host(dW).astype(np.float64)


def _exact(y, a, absolute=False):
    G = y.shape[0]
    if absolute:
        y, a = y & 0x7F, a & 0x7F
    yT = np.ascontiguousarray(y.transpose(1, 0, 2)).reshape(128, G * 128)
    aT = np.ascontiguousarray(a.transpose(1, 0, 2)).reshape(128, G * 128)
    s1 = np.ones((128, G), np.float32)
    return OG.grouped_wgrad(yT, s1, aT, s1, np.arange(G + 1))


def _rule_bound(y, a):
    """Bound implied by the truncation rule: per run of 8 tokens, every product
    but the largest loses less than one unit of 2^(floor(log2 max) - 13) (and
    never more than itself); plus the FP32 additions of 16 run sums (17
    roundings of the running total, at most 2^-24 of sum |p| each)."""
    yv, av = OF.e4m3_decode(y), OF.e4m3_decode(a)
    G = y.shape[0]
    out = np.zeros((G, 128, 128))
    mag = np.zeros((G, 128, 128))
    for r0 in range(0, 128, 8):
        p = np.abs(yv[:, :, None, r0:r0 + 8] * av[:, None, :, r0:r0 + 8])   # [G, n, k, 8]
        mx = p.max(axis=3)
        lsb = np.ldexp(1.0, np.floor(np.log2(np.where(mx > 0, mx, 1.0))).astype(int) - 13)
        out += np.minimum(p, lsb[..., None]).sum(axis=3) - np.minimum(mx, lsb)
        mag += p.sum(axis=3)
    return out + 17 * 2.0 ** -24 * mag


def _tiles(v, G):
    """1x128 quantisation of [G*128, 128] data (rows are columns of a chunk, the
    128 values run along its tokens) -> [G, 128, 128] codes."""
    q, _ = OQ.quant_1x128(np.asarray(v, np.float32))
    return q.reshape(G, 128, 128)


def test_mfma_truncation_rule():
    """Hand-built dot products (column 0 of both operands, other bytes 0):
    a small product is kept exactly when it is at most 13 binades below the
    largest product of its run of 8 tokens, dropped below that; truncation is
    toward zero; products in different runs are kept exactly."""
    enc = lambda v: OF.e4m3_encode(np.array([v], np.float64))[0]
    cases = []      # (terms [(token, y, a)], expected)
    for j in (13, 14):                       # 2^16 + 2^(16-j), same run
        cases.append(([(0, 256.0, 256.0), (1, 2.0 ** (8 - j), 256.0)],
                      65536.0 + (2.0 ** (16 - j) if j <= 13 else 0.0)))
    cases.append(([(0, 256.0, 256.0), (8, 1.0, 1.0)], 65537.0))                # next run
    cases.append(([(0, 256.0, 256.0), (7, 1.0, 1.0)], 65536.0))                # same run
    cases.append(([(0, 256.0, 256.0), (1, 1.75, 16.0)], 65536.0 + 24.0))       # 28 -> 24 (unit 8)
    cases.append(([(0, 256.0, 256.0), (1, -1.75, 16.0)], 65536.0 - 24.0))      # toward zero
    cases.append(([(0, 448.0, 448.0), (64, 1.0, 1.0)], 200705.0))             # second instruction
    G = len(cases)
    y = np.zeros((G, 128, 128), np.uint8)
    a = np.zeros((G, 128, 128), np.uint8)
    for g, (terms, _) in enumerate(cases):
        for tok, vy, va in terms:
            y[g, 0, tok], a[g, 0, tok] = enc(vy), enc(va)
    got = _wgrad_dots(y, a)[:, 0, 0]
    exp = np.array([e for _, e in cases])
    log("[mfma] rule cases: got " + " ".join(f"{v!r}" for v in got))
    assert np.array_equal(got, exp)


@pytest.mark.parametrize("dist", ["codes", "gaussian", "swiglu", "wide"])
def test_mfma_error_within_rule(dist):
    """Random 128-term dot products (64 groups x 128 x 128) stay within the
    bound the truncation rule implies, for operand distributions from
    uniformly random codes (a 2^18 range inside a tile) to Gaussian tiles."""
    G = 64
    rng = np.random.default_rng({"codes": 1, "gaussian": 2, "swiglu": 3, "wide": 4}[dist])
    if dist == "codes":
        c = rng.integers(0, 254, (2, G, 128, 128)).astype(np.uint8)
        y, a = np.where(c >= 0x7F, c + 1, c).astype(np.uint8)      # no NaN codes
    else:
        v = rng.standard_normal((2, G * 128, 128))
        if dist == "swiglu":
            g = 0.5 * rng.standard_normal(v.shape)
            v = g / (1 + np.exp(-g)) * v
        if dist == "wide":
            v = v * np.exp(2.0 * rng.standard_normal(v.shape))
        y, a = _tiles(v[0], G), _tiles(v[1], G)
    got = _wgrad_dots(y, a)
    err = np.abs(got - _exact(y, a))
    bound = _rule_bound(y, a)
    log(f"[mfma] {dist}: largest error / rule bound {np.max(err / np.maximum(bound, 1e-300)):.3f}")
    assert np.all(err <= bound)


def _block_rel(y, a):
    got = _wgrad_dots(y, a)
    mag = _exact(y, a, absolute=True)
    nz = mag > 0
    rel = np.abs(got - _exact(y, a))[nz] / mag[nz]
    return float(rel.max()), float(rel.mean())


def test_mfma_term_forward_operands():
    """The forward GEMMs' operands against 128x128 blocks of N(0, 1) weights:
    1x128 tiles of N(0, 1) data (x, the gate+up operand the GEMM bounds of
    the other tests are applied to) keep the block error within 2^-14 of the
    sum of |products| (MFMA_BLOCK_REL); 1x128 tiles of silu(g)*u (h, the
    down projection's operand, a wider range inside a tile) within 2^-13."""
    G = 128
    rng = np.random.default_rng(12)
    w = _tiles(rng.standard_normal((G * 128, 128)), G)
    x = _tiles(rng.standard_normal((G * 128, 128)), G)
    g = 0.5 * rng.standard_normal((G * 128, 128))
    h = _tiles(g / (1 + np.exp(-g)) * 0.5 * rng.standard_normal(g.shape), G)
    for name, op, lim in (("x", x, 2.0 ** -14), ("h", h, 2.0 ** -13)):
        mx, mean = _block_rel(op, w)
        log(f"[mfma] forward {name} x W: error / sum|p| max 2^{np.log2(mx):.2f}, mean 2^{np.log2(mean):.2f}")
        assert mx <= lim


def test_mfma_term_weight_gradient_operands():
    """The weight gradient's operands - 128x1 tiles (along tokens) of gate
    weight times output gradient and of SwiGLU outputs - keep the block error
    within 2^-12 of the sum of |products| (the wgrad bound's MFMA term)."""
    G = 128
    rng = np.random.default_rng(13)
    wdy = rng.uniform(0.05, 0.25, (G * 128, 1)) * rng.standard_normal((G * 128, 128))
    g = 0.5 * rng.standard_normal((G * 128, 128))
    h = g / (1 + np.exp(-g)) * 0.5 * rng.standard_normal(g.shape)
    mx, mean = _block_rel(_tiles(wdy, G), _tiles(h, G))
    log(f"[mfma] wgrad w*dy x h: error / sum|p| max 2^{np.log2(mx):.2f}, mean 2^{np.log2(mean):.2f}")
    assert mx <= 2.0 ** -12
