"""Backward for input of the expert GEMMs on the GPU, through the C ABI.

fp8_transpose_128x128 moves bytes and scales only, so it must equal the
oracle's block transpose bit for bit (random bytes, every code including
NaN patterns).  The input gradient dA = dY W is grouped_fp8_gemm on the
transposed blocks, or grouped_fp8_gemm_dgrad on W in its forward layout
(the same MFMA operand bytes in the same K positions, so the two agree bit
for bit on any data); with integer-valued E4M3 operands in [-2, 2] and
power-of-two scales 2^[-2, 2] every partial, scaled block and running sum is
exact in fp32 (|sum| < 2^19 on a 2^-4 grid for contractions up to 7168), so
the GPU's bf16 output must equal the oracle's bf16 rounding of the exact
gradient bit for bit.
"""
import numpy as np
import pytest
import torch

import synth
import fp8_block_scaled_bias_amd as M
from gpu_common import bf16_bits_host, bf16_values_host, dev, host, log
from oracle import formats as OF
from oracle import gemm as OG

pytestmark = pytest.mark.gpu

VALS = np.arange(-2, 3, dtype=np.float32)


def _codes(shape, seed):
    lut = OF.e4m3_encode(VALS)
    v = synth.int_fp8_operand(shape, seed, -2, 2)
    return lut[(v + 2).astype(np.int8)]


def _transpose_dev(w_d, ws_d, G, N, K):
    wt = torch.empty((G, K, N), dtype=torch.uint8, device="cuda")
    wts = torch.empty((G, K // 128, N // 128), dtype=torch.float32, device="cuda")
    M.fp8_transpose_128x128(w_d, ws_d, G, N, K, wt, wts)
    return wt, wts


@pytest.mark.parametrize("G,N,K", [(3, 256, 384), (1, 128, 128), (2, 1024, 128), (5, 384, 1280)])
def test_transpose_exact(G, N, K):
    rng = np.random.default_rng([G, N, K])
    w = rng.integers(0, 256, (G, N, K), dtype=np.uint8)
    ws = rng.random((G, N // 128, K // 128)).astype(np.float32)
    log(f"[transpose] G={G} N={N} K={K}")
    wt, wts = _transpose_dev(dev(w), dev(ws), G, N, K)
    qT, sT = OG.transpose_blocks(w, ws)
    assert np.array_equal(host(wt), qT)
    assert np.array_equal(host(wts), sT)


@pytest.mark.parametrize("N,K", [(4096, 7168), (7168, 2048)], ids=["w_gate_up", "w_down"])
def test_transpose_full_shape_sampled(N, K):
    """All 257 experts' weights at the layer's shapes (7.5 / 3.8 GB); the scales
    whole, 24 random blocks and the last block byte for byte."""
    G = 257
    log(f"[transpose] full G={G} N={N} K={K}")
    gen = torch.Generator(device="cuda").manual_seed(N + K)
    w_d = torch.randint(0, 256, (G, N, K), dtype=torch.uint8, device="cuda", generator=gen)
    ws_d = torch.rand((G, N // 128, K // 128), dtype=torch.float32, device="cuda", generator=gen)
    wt, wts = _transpose_dev(w_d, ws_d, G, N, K)
    torch.cuda.synchronize()
    _, sT = OG.transpose_blocks(np.zeros((1, 1, 1), np.uint8), host(ws_d))
    assert np.array_equal(host(wts), sT)
    rng = np.random.default_rng(7)
    picks = [(int(rng.integers(G)), int(rng.integers(N // 128)), int(rng.integers(K // 128))) for _ in range(24)]
    picks.append((G - 1, N // 128 - 1, K // 128 - 1))
    for g, nb, kb in picks:
        blk = host(w_d[g, nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128])
        got = host(wt[g, kb * 128:(kb + 1) * 128, nb * 128:(nb + 1) * 128])
        assert np.array_equal(got, OG.transpose_blocks(blk, np.zeros((1, 1), np.float32))[0]), (g, nb, kb)
    log(f"[transpose] full G={G} N={N} K={K}: scales whole and {len(picks)} blocks bit-exact")


def _dgrad_dev(path, qY_d, sY_d, w_d, ws_d, offs_d, G, Mt, N, K):
    out = torch.empty((Mt, K), dtype=torch.bfloat16, device="cuda")
    if path == "forward_layout":
        M.grouped_fp8_gemm_dgrad(qY_d, sY_d, w_d, ws_d, offs_d, G, Mt, N, K, out)
    else:
        wt, wts = _transpose_dev(w_d, ws_d, G, N, K)
        M.grouped_fp8_gemm(qY_d, sY_d, None, wt, wts, offs_d, G, Mt, K, N, out)
    return out


@pytest.mark.parametrize("rows,N,K", [
    ([300, 0, 77, 513, 129], 384, 512),      # small-group kernel, ragged groups, an empty one
    ([700, 410, 905, 262], 1536, 512),        # 256x256-tile kernel (contraction 12 blocks)
], ids=["small_tiles", "wide_tiles"])
def test_dgrad_exact(rows, N, K):
    """dA = dY W for groups of the forward C = A W^T (W [N, K]): the grouped GEMM
    on W^T from the transpose, against the oracle's block-scaled dgrad."""
    G = len(rows)
    offs = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    Mt = int(offs[-1])
    qY = _codes((Mt, N), 31 + N)
    sY = synth.pow2_scales((Mt, N // 128), 32 + N, -2, 2)
    qW = _codes((G, N, K), 33 + K)
    sW = synth.pow2_scales((G, N // 128, K // 128), 34 + K, -2, 2)
    log(f"[dgrad] rows {rows} N={N} K={K}")
    wt, wts = _transpose_dev(dev(qW), dev(sW), G, N, K)
    out = torch.empty((Mt, K), dtype=torch.bfloat16, device="cuda")
    M.grouped_fp8_gemm(dev(qY), dev(sY), None, wt, wts, dev(offs.astype(np.int32)), G, Mt, K, N, out)
    ref = OG.to_bf16(OG.grouped_dgrad(qY, sY, qW, sW, offs))
    got = bf16_values_host(out)
    assert np.array_equal(got, ref), int((got != ref).sum())


@pytest.mark.parametrize("rows,N,K", [
    ([300, 0, 77, 513, 129], 768, 512),      # 256x256 tiles: ragged groups, an empty one
    ([700, 410, 905, 262], 1536, 512),        # 256x256 tiles, 12 contraction blocks
    ([300, 0, 77, 513, 129], 384, 384),      # 128-row tiles; last column tile half full
    ([5, 40, 1, 290], 1024, 768),             # 64-row tiles
    ([3, 0, 17, 9, 30, 1], 256, 128),         # 32-row tiles; one half-full column tile
], ids=["wide_ragged", "wide", "bm128_half_cols", "bm64", "bm32_half_cols"])
def test_dgrad_forward_layout_exact(rows, N, K):
    """grouped_fp8_gemm_dgrad: dA = dY W read from W [N, K] as stored for the
    forward (no transposed copy), against the oracle's block-scaled dgrad, in
    every tile shape (rows per group choose it, as in grouped_fp8_gemm)."""
    G = len(rows)
    offs = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    Mt = int(offs[-1])
    qY = _codes((Mt, N), 51 + N)
    sY = synth.pow2_scales((Mt, N // 128), 52 + N, -2, 2)
    qW = _codes((G, N, K), 53 + K)
    sW = synth.pow2_scales((G, N // 128, K // 128), 54 + K, -2, 2)
    log(f"[dgrad fwd-layout] rows {rows} N={N} K={K}")
    out = _dgrad_dev("forward_layout", dev(qY), dev(sY), dev(qW), dev(sW),
                     dev(offs.astype(np.int32)), G, Mt, N, K)
    ref = OG.to_bf16(OG.grouped_dgrad(qY, sY, qW, sW, offs))
    got = bf16_values_host(out)
    assert np.array_equal(got, ref), int((got != ref).sum())


@pytest.mark.parametrize("rows,N,K", [([700, 0, 410, 905, 262], 2048, 1024),
                                      ([50, 7, 90, 33], 512, 640)], ids=["wide", "bm64"])
def test_dgrad_forward_layout_equals_transposed_random(rows, N, K):
    """On Gaussian data quantised 1x128 / 128x128 (inexact sums), the
    forward-layout dgrad and the grouped GEMM on the transposed blocks feed
    the MFMAs the same bytes in the same K positions: equal bit for bit."""
    from oracle import quant as OQ
    G = len(rows)
    offs = np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)
    Mt = int(offs[-1])
    rng = np.random.default_rng(61)
    qY, sY = OQ.quant_1x128(rng.standard_normal((Mt, N)).astype(np.float32))
    qW = np.empty((G, N, K), np.uint8)
    sW = np.empty((G, N // 128, K // 128), np.float32)
    for g in range(G):
        qW[g], sW[g] = OQ.quant_128x128((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    args = (dev(qY), dev(sY), dev(qW), dev(sW), dev(offs.astype(np.int32)), G, Mt, N, K)
    a = bf16_bits_host(_dgrad_dev("forward_layout", *args))
    b = bf16_bits_host(_dgrad_dev("transposed", *args))
    assert np.array_equal(a, b), int((a != b).sum())


def test_dgrad_forward_layout_rejects_bad_shape():
    """Output columns that are not a multiple of 128 are rejected before any
    launch with MOE_ERR_INVALID."""
    G, Mt, N, K = 2, 64, 768, 200
    y = torch.zeros((Mt, N), dtype=torch.uint8, device="cuda")
    ys = torch.ones((Mt, N // 128), dtype=torch.float32, device="cuda")
    w = torch.zeros((G, N, K), dtype=torch.uint8, device="cuda")
    ws = torch.ones((G, N // 128, K // 128), dtype=torch.float32, device="cuda")
    offs = torch.tensor([0, 32, 64], dtype=torch.int32, device="cuda")
    out = torch.empty((Mt, K), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(M.MoEError) as e:
        M.grouped_fp8_gemm_dgrad(y, ys, w, ws, offs, G, Mt, N, K, out)
    assert e.value.code == M._lib.MOE_ERR_INVALID


def _group_w(base, g):
    return np.roll(base.ravel(), 7919 * g).reshape(base.shape)


@pytest.mark.parametrize("path", ["transposed", "forward_layout"])
@pytest.mark.parametrize("N,K", [(7168, 2048), (4096, 7168)], ids=["down", "gate_up"])
def test_dgrad_full_shape_exact(N, K, path):
    """Input gradients of the layer's two expert GEMMs at T=16384 (147,456 rows
    in 257 groups: the routed counts of the prefill batch's multinomial stand-in
    plus the 16,384-row shared group): down's dH = dD W_dn (contraction 7168)
    and gate+up's dX = dGU W_gu (contraction 4096).  Sampled rows: the first,
    middle and last of every 16th group and of the last group."""
    G = 257
    counts = np.concatenate([synth.gen_group_counts(131072, G - 1, seed=0), [16384]])
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    R = int(offs[-1])
    log(f"[dgrad full] N={N} K={K}: R={R}")
    # dY row r is row r % 4093 of a random block (the oracle needs sampled rows only)
    ybase = _codes((4093, N), 41 + N)
    sY = synth.pow2_scales((R, N // 128), 42 + N, -2, 2)
    qY_d = torch.from_numpy(ybase).cuda()[torch.arange(R, device="cuda") % 4093]
    base = _codes((N, K), 43 + K)
    sW = synth.pow2_scales((G, N // 128, K // 128), 44 + K, -2, 2)
    base_d = torch.from_numpy(base).cuda().flatten()
    w_d = torch.empty((G, N, K), dtype=torch.uint8, device="cuda")
    for g in range(G):   # torch.roll matches np.roll (_group_w)
        w_d[g].copy_(torch.roll(base_d, 7919 * g).view(N, K))
    log(f"[dgrad full] N={N} K={K} {path}: launch")
    out = _dgrad_dev(path, qY_d, dev(sY), w_d, dev(sW), dev(offs.astype(np.int32)), G, R, N, K)
    torch.cuda.synchronize()
    del w_d
    checked = 0
    for g in list(range(0, G, 16)) + [G - 1]:
        r0, r1 = int(offs[g]), int(offs[g + 1])
        rws = sorted({r0, (r0 + r1) // 2, r1 - 1})
        got = bf16_values_host(out[rws])
        ref = OG.to_bf16(OG.block_scaled_dgrad(ybase[np.array(rws) % 4093], sY[rws], _group_w(base, g), sW[g]))
        assert np.array_equal(got, ref), (g, int((got != ref).sum()))
        checked += len(rws)
    log(f"[dgrad full] N={N} K={K}: {checked} sampled rows bit-exact")
