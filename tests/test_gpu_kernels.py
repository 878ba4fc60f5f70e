"""Per-kernel GPU parity against the oracle, through the C ABI.

Bars: bit-exact for codes, scales, indices, counts and permutations; the
GEMM is bit-exact on exactly representable data and within one bf16 ulp per
element otherwise (the oracle's sum is exact, the GPU's fp32 total differs by
rounding only, and one bf16 rounding follows); the combine likewise.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_common import (bf16_dev, bf16_values_host, bf16_ulp, dev, host, log, rel_l2, compare_routes,
                        assert_within_one_bf16_ulp)
from oracle import balance as OB
from oracle import combine as OC
from oracle import formats as OF
from oracle import gemm as OG
from oracle import permute as OP
from oracle import quant as OQ
from oracle import route as OR
from oracle import swiglu as OS

import fp8_block_scaled_bias_amd as M

pytestmark = pytest.mark.gpu


def _u8(shape):
    return torch.empty(shape, dtype=torch.uint8, device="cuda")


def _f32(shape):
    return torch.empty(shape, dtype=torch.float32, device="cuda")


def _i32(shape):
    return torch.empty(shape, dtype=torch.int32, device="cuda")


# ---------------------------------------------------------------- quantiser
def _quant_gpu(bits, K, ld, mode):
    Mrows = bits.shape[0]
    x = bf16_dev(bits)
    q, s = _u8((Mrows, K)), _f32((Mrows, K // 128))
    M.fp8_quant_1x128(x, Mrows, K, ld, mode, q, s)
    return host(q), host(s)


@pytest.mark.parametrize("rows,K", [(1, 128), (300, 1024), (77, 7168)])
def test_quant_identity_random(rows, K):
    rng = np.random.default_rng(rows + K)
    v = (rng.standard_normal((rows, K)) * np.exp(rng.uniform(-8, 8, (rows, 1)))).astype(np.float32)
    bits = synth.f32_to_bf16_bits(v)
    q, s = _quant_gpu(bits, K, K, 0)
    oq, os_ = OQ.quant_1x128(OF.bf16_value_from_bits(bits).astype(np.float32))
    assert np.array_equal(s, os_)
    assert np.array_equal(q, oq)


@pytest.mark.parametrize("arrangement", ["sorted", "shuffled"])
def test_quant_identity_every_bf16_pattern(arrangement):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    bits = bits[finite]
    if arrangement == "sorted":
        order = np.argsort(np.abs(OF.bf16_value_from_bits(bits)), kind="stable")
        bits = bits[order]
    else:
        bits = bits[np.random.default_rng(0).permutation(len(bits))]
    pad = (-len(bits)) % 1024
    bits = np.concatenate([bits, np.zeros(pad, np.uint16)]).reshape(-1, 1024)
    q, s = _quant_gpu(bits, 1024, 1024, 0)
    oq, os_ = OQ.quant_1x128(OF.bf16_value_from_bits(bits).astype(np.float32))
    assert np.array_equal(s, os_)
    assert np.array_equal(q, oq), int((q != oq).sum())


def test_quant_identity_strided_rows_and_zero_tiles():
    rows, K, ld = 40, 256, 384
    rng = np.random.default_rng(3)
    bits = synth.f32_to_bf16_bits(rng.standard_normal((rows, ld)).astype(np.float32))
    bits[5, :128] = 0
    bits[6, 128:256] = 0x8000       # negative zeros
    q, s = _quant_gpu(bits, K, ld, 0)
    oq, os_ = OQ.quant_1x128(OF.bf16_value_from_bits(bits[:, :K]).astype(np.float32))
    assert np.array_equal(s, os_) and np.array_equal(q, oq)
    assert s[5, 0] == 1.0 and np.all(q[6, 128:256] == 0x80)


@pytest.mark.parametrize("rows,I", [(257, 512), (64, 2048)])
def test_quant_swiglu(rows, I):
    rng = np.random.default_rng(rows)
    v = (rng.standard_normal((rows, 2 * I)) * 2).astype(np.float32)
    v[3, I:I + 128] = 0.0                               # u = 0 -> h = 0 tile
    bits = synth.f32_to_bf16_bits(v)
    q, s = _quant_gpu(bits, I, 2 * I, 1)
    oq, os_, h = OS.swiglu_quant(OF.bf16_value_from_bits(bits), I)
    # h is an fp32 chain with one exp; GPU and NumPy exp may differ in the
    # last ulp, which can move a scale by an ulp or a code across a rounding
    # midpoint by one step - nothing more.
    srel = np.abs(s.astype(np.float64) - os_) / os_
    assert srel.max() <= 2.0 ** -21, srel.max()
    diff = q != oq
    frac = diff.mean()
    log(f"[swiglu quant] rows {rows} I {I}: {int(diff.sum())} codes differ ({frac:.2e}), "
        f"scales differ in {int((s != os_).sum())} tiles")
    assert frac <= 1e-3
    a = OF.e4m3_decode(q[diff])
    b = OF.e4m3_decode(oq[diff])
    mags = OF.E4M3_TABLE[:0x7F]
    ia = np.searchsorted(mags, np.abs(a))
    ib = np.searchsorted(mags, np.abs(b))
    assert np.all(np.abs(ia - ib) <= 1) and np.all((np.sign(a) == np.sign(b)) | (a == 0) | (b == 0))
    assert np.all(s[3, 0] == 1.0) and np.all((q[3, :128] == 0) | (q[3, :128] == 0x80))


def test_quant_128x128_weights():
    G, N, K = 3, 256, 384
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((G, N, K)) * 0.006).astype(np.float32)
    w[1, 128:, :128] *= 1000
    w[2, :128, 256:] = 0
    q, s = _u8((G, N, K)), _f32((G, N // 128, K // 128))
    M.fp8_quant_128x128(dev(w), G, N, K, q, s)
    q, s = host(q), host(s)
    for g in range(G):
        oq, os_ = OQ.quant_128x128(w[g])
        assert np.array_equal(s[g], os_) and np.array_equal(q[g], oq)


def test_e4m3_conversion_every_boundary():
    # 128x128 fp32 blocks whose amax is exactly 448 have scale 1, so their
    # codes are E4M3(w) of the fp32 values themselves: every code value, every
    # midpoint between neighbours and the fp32 values next to it, subnormals,
    # signed zeros and random fp32 in [-448, 448]
    mags = OF.E4M3_TABLE[:0x7F]
    mids = 0.5 * (mags[:-1] + mags[1:])
    m32 = mids.astype(np.float32)
    vals = np.concatenate([mags, mids, np.nextafter(m32, np.float32(0)),
                           np.nextafter(m32, np.float32(1000)), [0.0, -0.0, 2.0 ** -10, 2.0 ** -11]])
    vals = np.concatenate([vals, -vals]).astype(np.float32)
    rng = np.random.default_rng(12)
    nblk = 8
    w = rng.uniform(-448, 448, (nblk * 128 * 128,)).astype(np.float32)
    w[:len(vals)] = vals
    w[len(vals):2 * len(vals)] = vals * np.float32(2.0 ** -7)   # into the subnormal grid
    w = w.reshape(nblk, 128, 128)
    w[:, 0, 0] = 448.0
    wt = np.ascontiguousarray(w.transpose(1, 0, 2).reshape(128, nblk * 128))   # [N=128, K]
    q, sc = _u8((1, 128, nblk * 128)), _f32((1, 1, nblk))
    M.fp8_quant_128x128(dev(wt[None]), 1, 128, nblk * 128, q, sc)
    oq, os_ = OQ.quant_128x128(wt)
    assert np.all(host(sc) == 1.0) and np.all(os_ == 1.0)
    assert np.array_equal(host(q)[0], oq), int((host(q)[0] != oq).sum())


# ------------------------------------------------------------------- router
def _route_gpu(bits, C, b, E, ng, tg, k):
    T, H = bits.shape
    idx, w, cnt, ts = _i32((T, k)), _f32((T, k)), _i32((E,)), _f32((T, k))
    wsb = max(16, M.moe_route_workspace_bytes(T, H, E))
    ws = _u8((wsb,))
    M.moe_route(bf16_dev(bits), T, H, dev(C), dev(b), E, ng, tg, k, idx, w, cnt, ws, wsb, topk_s=ts)
    ts = host(ts)
    # the weights are the chosen scores over their fp32 sum in slot order
    S = ts[:, 0].copy()
    for j in range(1, k):
        S = (S + ts[:, j]).astype(np.float32)
    assert np.array_equal(host(w), (ts / S[:, None]).astype(np.float32))
    return host(idx), host(w), host(cnt), ts


def _check_route(cfg, T, seed, label):
    bits = synth.gen_x(cfg, seed=seed, T=T)
    C = synth.gen_centroids(cfg, seed=seed)
    b = synth.gen_bias(cfg, seed=seed)
    idx, w, cnt, ts = _route_gpu(bits, C, b, cfg.E, cfg.n_group, cfg.topk_group, cfg.k)
    ora = OR.route(bits, C, b, cfg.n_group, cfg.topk_group, cfg.k)
    mism = compare_routes(idx, ora, label)
    ok = np.setdiff1d(np.arange(T), mism)
    # weights: fp32 sigmoid of fp32-accumulated logits vs float64, checked
    # relative to the oracle's weight (the bit-exact scope's reading: at most
    # 1e-6 relative)
    err = np.abs(w[ok].astype(np.float64) - ora["w"][ok])
    rel = err / ora["w"][ok]
    log(f"[route] {label}: max |w_gpu - w_oracle| = {err.max():.3e}, relative {rel.max():.3e}")
    assert rel.max() <= 1e-6
    # the chosen experts' unbiased scores (topk_s) to the same bar
    s_ref = np.take_along_axis(ora["s"][ok], idx[ok].astype(np.int64), axis=1)
    assert (np.abs(ts[ok].astype(np.float64) - s_ref) / s_ref).max() <= 1e-6
    assert np.array_equal(cnt, np.bincount(idx.ravel(), minlength=cfg.E))
    if len(mism) == 0:
        assert np.array_equal(cnt, ora["counts"])
    np.testing.assert_allclose(w.sum(axis=1), 1.0, atol=2e-6)
    return idx


def test_route_tiny():
    _check_route(synth.TINY, 64, 0, "tiny")


def test_route_mid_ragged():
    _check_route(synth.MID, 200, 1, "mid")
    _check_route(synth.MID.with_(n_group=1, topk_group=1), 77, 2, "mid-nogroup")


def test_route_v3_shapes():
    _check_route(synth.DECODE, 128, 0, "v3-T128")
    _check_route(synth.DECODE, 1000, 5, "v3-T1000")


# Large batches take the 256-token kernel with pre-split centroid planes:
# a ragged last token tile, fewer experts than the tile (E=64) and 4 or more
# K splits.
def test_route_large_batches():
    _check_route(synth.DECODE, 2100, 6, "v3-T2100")
    _check_route(synth.MID, 2500, 7, "mid-T2500")


def test_route_hand_traced_ties():
    from test_oracle_route import _ties_rows
    for E, ng, tg, k, b, ids, ws, _margin in _ties_rows():
        H = 256
        bits = np.zeros((70, H), np.uint16)
        C = synth.gen_centroids(synth.TINY.with_(E=E, H=H))
        idx, w, cnt, _ = _route_gpu(bits, C, b, E, ng, tg, k)
        assert np.all(idx == np.array(ids)), (idx[0], ids)
        assert np.all(w == np.array(ws, np.float32))
        exp = np.zeros(E, np.int64)
        exp[ids] = 70
        assert np.array_equal(cnt, exp)


def test_route_hand_traced_ties_large_batch():
    """The 256-expert hand-traced rows again on 2100 tokens of width 7168: the
    wide logits kernel with several K splits and the selection that prefetches
    the next token's partials.  Every score is exactly 1/2, so the threshold
    search ends on a shared score and the lowest expert ids fill the rest."""
    from test_oracle_route import _ties_rows
    T, H = 2100, 7168
    bits = np.zeros((T, H), np.uint16)
    for E, ng, tg, k, b, ids, ws, _margin in _ties_rows():
        if E != 256:
            continue
        C = synth.gen_centroids(synth.TINY.with_(E=E, H=H))
        idx, w, cnt, _ = _route_gpu(bits, C, b, E, ng, tg, k)
        assert np.all(idx == np.array(ids)), (idx[0], ids)
        assert np.all(w == np.array(ws, np.float32))
        exp = np.zeros(E, np.int64)
        exp[ids] = T
        assert np.array_equal(cnt, exp)
    log(f"[route] hand-traced ties on {T} tokens of width {H}: every token as traced")


def test_bias_update():
    rng = np.random.default_rng(4)
    for E, T, k in [(256, 4096, 8), (16, 64, 4), (256, 128, 8)]:
        counts = rng.multinomial(T * k, rng.dirichlet(np.ones(E))).astype(np.int32)
        counts[:3] = (T * k) // E if (T * k) % E == 0 else counts[:3]
        b = rng.uniform(-0.01, 0.01, E).astype(np.float32)
        bd = dev(b)
        M.moe_bias_update(dev(counts), bd, E, 0.001)
        assert np.array_equal(host(bd), OB.bias_update(counts, b, 0.001))


# -------------------------------------------------------------- permutation
def _permute_gpu(idx, E, ns, H=None, xq=None, xs=None):
    T, k = idx.shape
    counts = np.bincount(idx.ravel(), minlength=E).astype(np.int32)
    R = T * k + ns * T
    off, ps, inv = _i32((E + ns + 1,)), _i32((max(R, 1),)), _i32((max(T * k, 1),))
    wsb = max(16, M.moe_permute_workspace_bytes(T, k, E))
    ws = _u8((wsb,))
    a_out = a_s = None
    if xq is not None:
        a_out, a_s = _u8((R, H)), _f32((R, H // 128))
    M.moe_permute(dev(idx), dev(counts), T, k, E, ns, off, ps, inv,
                  dev(xq) if xq is not None else None, dev(xs) if xs is not None else None,
                  H or 128, a_out, a_s, ws, wsb)
    res = [host(off), host(ps)[:R], host(inv)[:T * k]]
    if xq is not None:
        res += [host(a_out), host(a_s)]
    return res


@pytest.mark.parametrize("T,k,E", [(1, 1, 4), (63, 4, 16), (200, 8, 64), (4097, 8, 256)])
def test_permute_random(T, k, E):
    rng = np.random.default_rng(T)
    idx = np.stack([np.sort(rng.choice(E, k, replace=False)) for _ in range(T)]).astype(np.int32)
    for ns in (0, 1):
        off, ps, inv = _permute_gpu(idx, E, ns)
        o_off, o_ps, o_inv = OP.permute(idx, E, ns)
        assert np.array_equal(off, o_off) and np.array_equal(ps, o_ps) and np.array_equal(inv, o_inv)


def test_permute_skewed_and_gather():
    T, k, E, H = 130, 2, 8, 256
    idx = np.tile(np.array([[1, 6]], np.int32), (T, 1))       # two experts take everything
    idx[7] = [0, 6]
    rng = np.random.default_rng(9)
    xq = rng.integers(0, 255, (T, H), dtype=np.uint8)
    xs = rng.standard_normal((T, H // 128)).astype(np.float32)
    off, ps, inv, a, a_s = _permute_gpu(idx, E, 1, H, xq, xs)
    o_off, o_ps, o_inv = OP.permute(idx, E, 1)
    assert np.array_equal(off, o_off) and np.array_equal(ps, o_ps) and np.array_equal(inv, o_inv)
    assert np.array_equal(a, xq[o_ps]) and np.array_equal(a_s, xs[o_ps])


# --------------------------------------------------------------------- GEMM
def _gemm_gpu(qA, sA, rowidx, qB, sB, offsets, N, K):
    Mt = int(offsets[-1])
    G = len(offsets) - 1
    C = torch.empty((Mt, N), dtype=torch.bfloat16, device="cuda")
    M.grouped_fp8_gemm(dev(qA), dev(sA), dev(rowidx) if rowidx is not None else None,
                       dev(qB), dev(sB), dev(offsets.astype(np.int32)), G, Mt, N, K, C)
    return bf16_values_host(C)


# Error of one FP8 MFMA 128-term partial relative to its absolute sum
# sum|a b|: gfx950's FP8 instructions truncate each product of a run of 8
# consecutive K positions to 13 binades below the run's largest product
# (pinned in test_gpu_mfma_precision).  On 1x128 tiles of Gaussian data and
# of SwiGLU outputs against 128x128 Gaussian weight blocks (the operands of
# these tests) the error reaches 2^-15.8 and 2^-14.1 of the absolute sum
# (test_mfma_term_forward_operands asserts 2^-14); uniformly random codes,
# which these tests never feed, reach 2^-12.2.
MFMA_BLOCK_REL = 2.0 ** -14
PROMO_ROUNDINGS = 5


def gemm_accumulation_bound(qA, sA, qB, sB, offsets, K):
    """Bound on |GPU fp32 total - exact| per output: each K block's MFMA
    partial is off by at most MFMA_BLOCK_REL of its absolute sum, and each of
    the K/128 promotion steps rounds a few times relative to the running
    total, which never exceeds S = sum_kb |sA sB| sum_k |a b|: the
    zero-started form rounds the scale product and the FMA (2); the rescaled
    form the two scale products and their quotient, the multiply and the
    MFMA's add of the rescaled accumulator (4 on the sums' scale, 5 with the
    final multiply).  PROMO_ROUNDINGS = 5 covers both."""
    qBabs = [np.asarray(q) & 0x7F for q in qB]
    S = OG.grouped_gemm(np.asarray(qA) & 0x7F, sA, qBabs, sB, offsets)
    return (MFMA_BLOCK_REL + PROMO_ROUNDINGS * (K // 128 + 1) * 2.0 ** -24) * S


@pytest.mark.parametrize("with_index", [False, True])
def test_gemm_integer_exact(with_index):
    sizes = [0, 1, 130, 257, 64, 0, 128]
    G, N, K = len(sizes), 256, 384
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    Mt = int(offsets[-1])
    rows_src = 300 if with_index else Mt
    A = synth.int_fp8_operand((rows_src, K), 1)
    qA = OF.e4m3_encode(A)
    sA = synth.pow2_scales((rows_src, K // 128), 2, -2, 2)
    B = synth.int_fp8_operand((G, N, K), 3)
    qB = OF.e4m3_encode(B)
    sB = synth.pow2_scales((G, N // 128, K // 128), 4, -2, 2)
    rowidx = np.random.default_rng(5).integers(0, rows_src, Mt).astype(np.int32) if with_index else None
    got = _gemm_gpu(qA, sA, rowidx, qB, sB, offsets, N, K)
    qAr = qA[rowidx] if with_index else qA
    sAr = sA[rowidx] if with_index else sA
    ref = OG.to_bf16(OG.grouped_gemm(qAr, sAr, qB, sB, offsets))
    assert np.array_equal(got, ref), int((got != ref).sum())


def _int_gemm_case(sizes, N, K, rows_src, seed):
    G = len(sizes)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    Mt = int(offsets[-1])
    A = synth.int_fp8_operand((rows_src, K), seed)
    qA = OF.e4m3_encode(A)
    sA = synth.pow2_scales((rows_src, K // 128), seed + 1, -2, 2)
    qB = OF.e4m3_encode(synth.int_fp8_operand((G, N, K), seed + 2))
    sB = synth.pow2_scales((G, N // 128, K // 128), seed + 3, -2, 2)
    return offsets, Mt, qA, sA, qB, sB


# Many tiles per persistent workgroup (tile loop and cross-tile copy
# pipeline), each M-tile configuration (rows per group ~5 -> 32, ~60 -> 64,
# ~2000 -> 128), with and without row gather, and the single-K-block case.
@pytest.mark.parametrize("mean_rows,G,N,K", [(2000, 20, 512, 384), (60, 300, 256, 256),
                                             (5, 257, 256, 256), (700, 40, 384, 128)])
@pytest.mark.parametrize("with_index", [False, True])
def test_gemm_integer_exact_many_tiles(mean_rows, G, N, K, with_index):
    rng = np.random.default_rng(mean_rows + G)
    sizes = rng.multinomial(mean_rows * G, np.full(G, 1.0 / G)).tolist()
    sizes[1] = 0
    rows_src = 3001 if with_index else int(sum(sizes))
    offsets, Mt, qA, sA, qB, sB = _int_gemm_case(sizes, N, K, rows_src, 7 + G)
    rowidx = rng.integers(0, rows_src, Mt).astype(np.int32) if with_index else None
    got = _gemm_gpu(qA, sA, rowidx, qB, sB, offsets, N, K)
    qAr = qA[rowidx] if with_index else qA
    sAr = sA[rowidx] if with_index else sA
    ref = OG.to_bf16(OG.grouped_gemm(qAr, sAr, qB, sB, offsets))
    assert np.array_equal(got, ref), int((got != ref).sum())


# Large groups (256x256 tiles, taken for an even number of >= 4 K blocks):
# every remainder class of the last M tile (1..64, 65..128, 129..192,
# 193..256 rows), empty groups, 6 to 12 K blocks (6: no interior steps
# between a tile's first 4 and last 8), with and without row gather.
@pytest.mark.parametrize("K", [768, 1024, 1536])
@pytest.mark.parametrize("with_index", [False, True])
def test_gemm_integer_exact_wide(K, with_index):
    sizes = [1000, 0, 170, 400, 256, 513, 65, 129, 200, 0, 700]
    N = 512
    rng = np.random.default_rng(K)
    rows_src = 2222 if with_index else int(sum(sizes))
    offsets, Mt, qA, sA, qB, sB = _int_gemm_case(sizes, N, K, rows_src, 31 + K)
    rowidx = rng.integers(0, rows_src, Mt).astype(np.int32) if with_index else None
    got = _gemm_gpu(qA, sA, rowidx, qB, sB, offsets, N, K)
    qAr = qA[rowidx] if with_index else qA
    sAr = sA[rowidx] if with_index else sA
    ref = OG.to_bf16(OG.grouped_gemm(qAr, sAr, qB, sB, offsets))
    assert np.array_equal(got, ref), int((got != ref).sum())


# Collapsed routing: a few groups hold every row, the rest are empty (the
# 256x256-tile kernel's cost-balanced ranges over very uneven groups).
@pytest.mark.parametrize("with_index", [False, True])
def test_gemm_integer_exact_collapsed(with_index):
    G, N, K = 65, 512, 1024
    sizes = [0] * G
    for g in (3, 17, 18, 40, 41, 42, 60, 63):
        sizes[g] = 2048
    sizes[G - 1] = 2048
    rng = np.random.default_rng(11)
    rows_src = 2048 if with_index else int(sum(sizes))
    offsets, Mt, qA, sA, qB, sB = _int_gemm_case(sizes, N, K, rows_src, 57)
    rowidx = np.tile(np.arange(2048, dtype=np.int32), 9) if with_index else None
    got = _gemm_gpu(qA, sA, rowidx, qB, sB, offsets, N, K)
    qAr = qA[rowidx] if with_index else qA
    sAr = sA[rowidx] if with_index else sA
    ref = OG.to_bf16(OG.grouped_gemm(qAr, sAr, qB, sB, offsets))
    assert np.array_equal(got, ref), int((got != ref).sum())


# Gathered row indices outside [0, A_rows) read row A_rows - 1 (documented
# clamp; the copies never leave A).  Small-group and 256-row-tile kernels.
@pytest.mark.parametrize("sizes", [[40, 7, 90], [300, 200, 0, 260]])
def test_gemm_gather_index_clamped(sizes):
    N, K, rows_src = 256, 1024, 50
    offsets, Mt, qA, sA, qB, sB = _int_gemm_case(sizes, N, K, rows_src, 7)
    rng = np.random.default_rng(3)
    rowidx = rng.integers(-5, rows_src + 20, Mt).astype(np.int32)
    rowidx[:3] = [-2**31, 2**31 - 1, rows_src]
    got = _gemm_gpu(qA, sA, rowidx, qB, sB, offsets, N, K)
    clamped = np.where((rowidx < 0) | (rowidx >= rows_src), rows_src - 1, rowidx)
    ref = OG.to_bf16(OG.grouped_gemm(qA[clamped], sA[clamped], qB, sB, offsets))
    assert np.array_equal(got, ref), int((got != ref).sum())


def test_gemm_swiglu_exact_sums_small_groups():
    """Fused gate+up launches with a handful of rows per group (fewer than 40
    on average: the decode regime, 32-row tiles, bound by the weight stream)
    take the exact-sum MFMA form (eight instructions per K block, one K
    position of every run of 8 in each) in tiles of more than 16 rows: their
    fp32 gate/up totals are the exact block-scaled sums up to fp32
    roundings, so every E4M3 code of h is the oracle's unless h lies within
    those roundings of a rounding midpoint (check_fused_swiglu with the
    fp32-rounding bound: 8 phase additions and the promotion per K block).
    Rows of tiles of at most 16 rows (groups 5, 1, 3, 9, 2, 12 and the last
    8 rows of the 40) keep the single-instruction form and its MFMA bound."""
    sizes = [5, 0, 31, 1, 17, 3, 40, 9, 2, 12]
    G, K, I, BM = len(sizes), 1024, 256, 32
    N = 2 * I
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    Mt = int(offsets[-1])
    rng = np.random.default_rng(78)
    qA, sA = OQ.quant_1x128(rng.standard_normal((Mt, K)).astype(np.float32))
    qB = np.empty((G, N, K), np.uint8)
    sB = np.empty((G, N // 128, K // 128), np.float32)
    for g in range(G):
        qB[g], sB[g] = OQ.quant_128x128((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    exact = OG.grouped_gemm(qA, sA, qB, sB, offsets)
    S = OG.grouped_gemm(qA & 0x7F, sA, [q & 0x7F for q in qB], sB, offsets)
    big = np.zeros(Mt, bool)
    for g, m in enumerate(sizes):
        for m0 in range(0, m, BM):
            if min(BM, m - m0) > 16:
                big[offsets[g] + m0:offsets[g] + min(m, m0 + BM)] = True
    assert big.sum() == 31 + 17 + 32
    bound = gemm_accumulation_bound(qA, sA, qB, sB, offsets, K)
    bound[big] = (10 * (K // 128) + 2) * 2.0 ** -24 * S[big]
    q, sc = _swiglu_gpu(qA, sA, None, qB, sB, offsets, I, K)
    n = check_fused_swiglu(q[big], sc[big], exact[big], bound[big], I, "exact-sum SwiGLU")
    check_fused_swiglu(q[~big], sc[~big], exact[~big], bound[~big], I, "single-form SwiGLU")
    log(f"[gemm exact] SwiGLU codes of exact-form tiles differing from the oracle: {n} of "
        f"{q[big].size}")


@pytest.mark.parametrize("sizes,N,K", [([5, 0, 300, 129], 384, 1024), ([1000], 256, 7168),
                                       ([700, 300, 0, 450], 512, 2048)])
def test_gemm_random_within_one_ulp(sizes, N, K):
    G = len(sizes)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    Mt = int(offsets[-1])
    rng = np.random.default_rng(Mt)
    a = rng.standard_normal((Mt, K)).astype(np.float32)
    qA, sA = OQ.quant_1x128(a)
    qB = np.empty((G, N, K), np.uint8)
    sB = np.empty((G, N // 128, K // 128), np.float32)
    for g in range(G):
        qB[g], sB[g] = OQ.quant_128x128((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    got = _gemm_gpu(qA, sA, None, qB, sB, offsets, N, K)
    exact = OG.grouped_gemm(qA, sA, qB, sB, offsets)
    ref = OG.to_bf16(exact)
    assert_within_one_bf16_ulp(got, ref, f"gemm {sizes} N={N} K={K}",
                               gemm_accumulation_bound(qA, sA, qB, sB, offsets, K))
    assert rel_l2(got, exact) < 3e-3


def _swiglu_gpu(qA, sA, rowidx, qB, sB, offsets, I, K):
    Mt = int(offsets[-1])
    G = len(offsets) - 1
    hq, hs = _u8((Mt, I)), _f32((Mt, I // 128))
    M.grouped_fp8_gemm_swiglu(dev(qA), dev(sA), dev(rowidx) if rowidx is not None else None,
                              dev(qB), dev(sB), dev(offsets.astype(np.int32)), G, Mt, I, K, hq,
                              hs)
    return host(hq), host(hs)


def check_fused_swiglu(q, s, exact, bound, I, what):
    """Compare GPU codes/scales with the oracle's fused reading.

    exact, bound: float64 [M, 2I] exact GEMM sums and the bound on the GPU's
    deviation from them.  h = silu(g) u moves by at most
    dh = |u| |silu'(g)| Bg + |silu(g)| Bu (+ fp32 rounding); a tile's scale by
    at most max(dh)/448; a code may differ only by one step, and only where
    the oracle's h/s lies within that movement of a rounding midpoint.
    """
    oq, os_, oh = OS.swiglu_quant(exact, I)
    g, u = exact[:, :I], exact[:, I:]
    Bg, Bu = bound[:, :I], bound[:, I:]
    sig = 1.0 / (1.0 + np.exp(-g))
    dsilu = sig * (1.0 + g * (1.0 - sig))
    # + fp32 evaluation of h: the kernel takes exp as 2^(g * -log2 e) on the
    # hardware exp2 (the rounded argument moves exp by |g| 2^-24 relative) and
    # uses the hardware reciprocal; a few ulp more
    dh = (np.abs(u) * np.abs(dsilu) * Bg + np.abs(g * sig) * Bu
          + (np.abs(g) + 8.0) * 2.0 ** -23 * np.abs(oh))
    Mt = exact.shape[0]
    dh_t = dh.reshape(Mt, I // 128, 128).max(axis=2)
    s_tol = dh_t / 448.0 + 2.0 ** -22 * os_
    sdiff = np.abs(s.astype(np.float64) - os_)
    assert np.all(sdiff <= s_tol), f"{what}: scale off by {(sdiff / s_tol).max():.2f}x the bound"
    diff = q != oq
    n = int(diff.sum())
    log(f"[{what}] codes differing: {n} of {q.size} ({n / q.size:.2e}); scales differing: "
        f"{int((s != os_).sum())} of {s.size}")
    if n:
        # each differing GPU code must be the E4M3 rounding of some value
        # within the derived movement of the oracle's h/s
        rows, cols = np.nonzero(diff)
        sc = np.repeat(os_, 128, axis=1)[rows, cols]
        v = oh[rows, cols].astype(np.float64) / sc
        got = OF.e4m3_decode(q[rows, cols])
        av = np.abs(v)
        quantum = np.where(av < 2.0 ** -6, 2.0 ** -9,
                           np.ldexp(1.0, np.floor(np.log2(np.maximum(av, 2.0 ** -6))).astype(int) - 3))
        slack = dh[rows, cols] / sc + av * (s_tol[rows, cols // 128] / sc) + 2.0 ** -20 * av
        err = np.abs(got - v)
        ok = err <= 0.5 * quantum * (1 + 1e-9) + 2 * slack + 1e-12
        assert np.all(ok), f"{what}: {int((~ok).sum())} codes outside the bound"
    return n


@pytest.mark.parametrize("sizes,I,K,with_index", [([5, 0, 300, 129], 256, 1024, False),
                                                  ([3, 40, 1], 384, 256, True),
                                                  ([1000], 128, 7168, False),
                                                  ([2500] * 12, 256, 384, True),
                                                  ([6] * 200, 256, 256, True),
                                                  ([300, 0, 77, 513], 256, 768, True),
                                                  ([600, 190], 384, 1024, False)])
def test_gemm_swiglu_fused(sizes, I, K, with_index):
    G = len(sizes)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    Mt = int(offsets[-1])
    rng = np.random.default_rng(Mt + I)
    rows_src = 77 if with_index else Mt
    qA, sA = OQ.quant_1x128(rng.standard_normal((rows_src, K)).astype(np.float32))
    rowidx = rng.integers(0, rows_src, Mt).astype(np.int32) if with_index else None
    qB = np.empty((G, 2 * I, K), np.uint8)
    sB = np.empty((G, 2 * I // 128, K // 128), np.float32)
    for g in range(G):
        qB[g], sB[g] = OQ.quant_128x128((rng.standard_normal((2 * I, K)) * 0.05).astype(np.float32))
    q, s = _swiglu_gpu(qA, sA, rowidx, qB, sB, offsets, I, K)
    Ar = qA[rowidx] if with_index else qA
    sAr = sA[rowidx] if with_index else sA
    exact = OG.grouped_gemm(Ar, sAr, qB, sB, offsets)
    bound = gemm_accumulation_bound(Ar, sAr, qB, sB, offsets, K)
    check_fused_swiglu(q, s, exact, bound, I, f"fused swiglu {sizes} I={I} K={K}")


# The fused gate+up that also keeps its bf16 outputs: codes and scales equal
# the fused kernel's, the kept outputs equal the plain GEMM's, bit for bit
# (256-row kernel: groups of >= 160 rows on average; smaller groups take the
# fused kernel and the plain GEMM in turn).
@pytest.mark.parametrize("sizes,with_index", [([1000, 0, 170, 400, 256, 513, 65], False),
                                              ([1000, 0, 170, 400, 256, 513, 65], True),
                                              ([5, 0, 300, 129], False)])
def test_gemm_swiglu_keep(sizes, with_index):
    import torch
    I, K = 256, 1024
    G = len(sizes)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    Mt = int(offsets[-1])
    rng = np.random.default_rng(Mt + 5)
    rows_src = 333 if with_index else Mt
    qA, sA = OQ.quant_1x128(rng.standard_normal((rows_src, K)).astype(np.float32))
    rowidx = rng.integers(0, rows_src, Mt).astype(np.int32) if with_index else None
    qB = np.empty((G, 2 * I, K), np.uint8)
    sB = np.empty((G, 2 * I // 128, K // 128), np.float32)
    for g in range(G):
        qB[g], sB[g] = OQ.quant_128x128((rng.standard_normal((2 * I, K)) * 0.05).astype(np.float32))
    args = (dev(qA), dev(sA), None if rowidx is None else dev(rowidx), dev(qB), dev(sB),
            dev(offsets.astype(np.int32)), G, Mt, I, K)
    hq, hs = _u8((Mt, I)), _f32((Mt, I // 128))
    M.grouped_fp8_gemm_swiglu(*args, hq, hs)
    kq, ks = _u8((Mt, I)), _f32((Mt, I // 128))
    gu = torch.full((Mt, 2 * I), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.grouped_fp8_gemm_swiglu_keep(*args, kq, ks, gu)
    plain = torch.full((Mt, 2 * I), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.grouped_fp8_gemm(dev(qA), dev(sA), None if rowidx is None else dev(rowidx), dev(qB), dev(sB),
                       dev(offsets.astype(np.int32)), G, Mt, 2 * I, K, plain)
    torch.cuda.synchronize()
    assert np.array_equal(host(kq), host(hq)) and np.array_equal(host(ks).view(np.uint32),
                                                                 host(hs).view(np.uint32))
    assert torch.equal(gu.view(torch.int16), plain.view(torch.int16))


# ------------------------------------------------------------------ combine
@pytest.mark.parametrize("shared", [True, False])
def test_combine(shared):
    T, k, H = 100, 8, 1024 + 512
    rng = np.random.default_rng(7)
    R = T * k + T
    Dbits = synth.f32_to_bf16_bits(rng.standard_normal((R, H)).astype(np.float32))
    inv = rng.permutation(T * k).astype(np.int32)
    w = rng.uniform(0.01, 1, (T, k)).astype(np.float32)
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    Dd = bf16_dev(Dbits)
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    M.moe_combine(Dd, dev(inv), dev(w), Dd[T * k:] if shared else None, T, k, H, y)
    got = bf16_values_host(y)
    Dv = OF.bf16_value_from_bits(Dbits)
    ref, ref64 = OC.combine(Dv, inv, w, T, k, Dv[T * k:] if shared else None)
    # fp32 sum of k+1 terms in slot order: |error| <= (k+1) 2^-24 sum |terms|
    _, absum = OC.combine(np.abs(Dv), inv, w, T, k, np.abs(Dv[T * k:]) if shared else None)
    assert_within_one_bf16_ulp(got, ref, "combine", (k + 1) * 2.0 ** -24 * absum)
    assert rel_l2(got, ref) < 1e-3
