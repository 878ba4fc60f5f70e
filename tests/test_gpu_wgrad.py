"""Weight gradient of the expert GEMMs on the GPU, through the C ABI.

The library keeps the 128x1-quantised operands chunk-major ([chunk, column,
128 tokens]); the oracle's are the logical transposed matrices [column,
tokens]: the tests convert between the two (_to_logical, _to_chunks).

fp8_quant_128x1_grouped must equal the oracle's grouped 128x1 quantiser
byte for byte (codes and scales: every decision is taken in fp32 on both
sides).  grouped_fp8_wgrad on integer-valued E4M3 codes in [-2, 2] with
power-of-two scales 2^[-2, 2] is exact in fp32 (128-token partials
|p| <= 512, scaled chunks multiples of 2^-4 below 2^13, totals within 2^20
for up to 128 chunks per group: 24 bits), so its fp32 output must equal the oracle's exact gradient bit for
bit.  On random data the two differ only by the GPU's fp32 accumulation: one
rounding of the scaled partial per chunk.
"""
import numpy as np
import pytest
import torch

import synth
import fp8_block_scaled_bias_amd as M
from gpu_common import dev, host, log
from oracle import formats as OF
from oracle import gemm as OG
from oracle import quant as OQ

pytestmark = pytest.mark.gpu

VALS = np.arange(-2, 3, dtype=np.float32)


def _codes(shape, seed):
    lut = OF.e4m3_encode(VALS)
    v = synth.int_fp8_operand(shape, seed, -2, 2)
    return lut[(v + 2).astype(np.int8)]


def _offsets(rows):
    return np.concatenate([[0], np.cumsum(rows)]).astype(np.int64)


def _to_logical(q_c, s_c, nch):
    """chunk-major [cap, C, 128] codes, [cap, C] scales -> [C, 128 nch], [C, nch]"""
    C = q_c.shape[1]
    return (np.ascontiguousarray(q_c[:nch].transpose(1, 0, 2)).reshape(C, nch * 128),
            np.ascontiguousarray(s_c[:nch].T))


def _to_chunks(q, s):
    """logical [C, 128 cap], [C, cap] -> chunk-major [cap, C, 128], [cap, C]"""
    C, P = q.shape
    return (np.ascontiguousarray(q.reshape(C, P // 128, 128).transpose(1, 0, 2)),
            np.ascontiguousarray(s.T))


def _quant_dev(x_bits, offs, G, C):
    Mt = x_bits.shape[0]
    cap = M.wgrad_chunks(Mt, G)
    q = torch.zeros((cap, C, 128), dtype=torch.uint8, device="cuda")
    s = torch.zeros((cap, C), dtype=torch.float32, device="cuda")
    xb = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).cuda().view(torch.bfloat16)
    M.fp8_quant_128x1_grouped(xb, C, None, dev(offs.astype(np.int32)), G, Mt, C, q, s, cap)
    return q, s, cap


@pytest.mark.parametrize("rows,C", [([300, 0, 77, 513, 129], 256), ([1], 128), ([128, 256, 5, 0], 384)])
def test_quant_128x1_grouped_exact(rows, C):
    offs = _offsets(rows)
    G, Mt = len(rows), int(offs[-1])
    bits = synth.gen_gemm_activations(Mt, C, seed=len(rows) + C)
    bits[:: 7, 3] = 0                                      # zeros inside tiles
    log(f"[quant128x1] rows {rows} C={C}")
    q, s, cap = _quant_dev(bits, offs, G, C)
    qo, so = OQ.quant_128x1_grouped(OF.bf16_value_from_bits(bits).astype(np.float32), offs)
    ql, sl = _to_logical(host(q), host(s), qo.shape[1] // 128)
    assert np.array_equal(ql, qo)
    assert np.array_equal(sl, so)


@pytest.mark.parametrize("rows,N,K", [([300, 0, 77, 513, 129], 256, 384), ([2000, 1100], 128, 256)],
                         ids=["ragged", "long_groups"])
def test_wgrad_exact(rows, N, K):
    offs = _offsets(rows)
    G, Mt = len(rows), int(offs[-1])
    cap = M.wgrad_chunks(Mt, G)
    pref = OQ.chunk_prefix(offs)
    qY = _codes((N, 128 * cap), 51 + N)
    qA = _codes((K, 128 * cap), 52 + K)
    sY = synth.pow2_scales((N, cap), 53, -2, 2)
    sA = synth.pow2_scales((K, cap), 54, -2, 2)
    log(f"[wgrad] rows {rows} N={N} K={K} chunks {cap}")
    dW = torch.full((G, N, K), float("nan"), dtype=torch.float32, device="cuda")
    (qYc, sYc), (qAc, sAc) = _to_chunks(qY, sY), _to_chunks(qA, sA)
    M.grouped_fp8_wgrad(dev(qYc), dev(sYc), dev(qAc), dev(sAc), cap, dev(offs.astype(np.int32)), G, Mt,
                        N, K, dW)
    ref = OG.grouped_wgrad(qY, sY, qA, sA, pref).astype(np.float32)
    got = host(dW)
    assert np.array_equal(got, ref), int((got != ref).sum())


def test_wgrad_random_end_to_end():
    """Quantise dY [M, N] and A [M, K] (bf16) on the GPU, then the gradient; against
    the oracle's quantiser (bit-exact codes) and exact gradient.  The bound is the
    grouped GEMM's: gfx950's FP8 MFMA returns a 128-term dot product within
    2^-14 of sum |products| (measured: mean 2^-19.4, max 2^-15.6, unbiased), and
    the promotion rounds twice per chunk (scale product, FMA), so
    |err| <= (2^-14 + 2 (chunks + 1) 2^-24) * S, S = sum_c |sY sA| sum |y a|.
    A wrong chunk, scale or row gives errors of the order of the values.  The
    MFMA's unbiased error, amplified by the cancellation in these random-sign
    sums, puts the relative L2 error near 1e-5 (checked below 1e-4)."""
    rows = [700, 0, 333, 129, 1024]
    offs = _offsets(rows)
    G, Mt, N, K = len(rows), int(offs[-1]), 256, 384
    yb = synth.gen_gemm_activations(Mt, N, seed=61)
    ab = synth.gen_gemm_activations(Mt, K, seed=62)
    qY, sY, cap = _quant_dev(yb, offs, G, N)
    qA, sA, _ = _quant_dev(ab, offs, G, K)
    dW = torch.empty((G, N, K), dtype=torch.float32, device="cuda")
    M.grouped_fp8_wgrad(qY, sY, qA, sA, cap, dev(offs.astype(np.int32)), G, Mt, N, K, dW)
    qYo, sYo = OQ.quant_128x1_grouped(OF.bf16_value_from_bits(yb).astype(np.float32), offs)
    qAo, sAo = OQ.quant_128x1_grouped(OF.bf16_value_from_bits(ab).astype(np.float32), offs)
    pref = OQ.chunk_prefix(offs)
    ref = OG.grouped_wgrad(qYo, sYo, qAo, sAo, pref)
    # the sum of |scaled partials| bounds the accumulation error: the MFMA's
    # partial error plus, per chunk, the rescaled accumulator's roundings (two
    # scale quotients, their product, the multiply, the MFMA's add) and the
    # final scale product and multiply: 6 (chunks + 1) roundings cover them
    Yd = np.abs(OQ.dequant_1x128(qYo, sYo))
    Ad = np.abs(OQ.dequant_1x128(qAo, sAo))
    got = host(dW).astype(np.float64)
    worst = 0.0
    for g in range(G):
        nch = int(pref[g + 1] - pref[g])
        cs = slice(int(pref[g]) * 128, int(pref[g + 1]) * 128)
        bound = (2.0 ** -14 + 6 * (nch + 1) * 2.0 ** -24) * (Yd[:, cs] @ Ad[:, cs].T) + 1e-30
        assert (np.abs(got[g] - ref[g]) <= bound).all(), g
        worst = max(worst, float(np.max(np.abs(got[g] - ref[g]) / bound)))
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    assert rel < 1e-4, rel
    log(f"[wgrad random] rel L2 {rel:.3e}; largest error / bound {worst:.3f}")


@pytest.mark.parametrize("N,K", [(7168, 2048), (4096, 7168)], ids=["down", "gate_up"])
def test_wgrad_full_shape_sampled(N, K):
    """The layer's two weight gradients at T=16384 (147,456 rows in 257 groups:
    multinomial routed counts + the 16,384-row shared group); dW is 15 / 30 GB of
    fp32.  Exact integer operands (row r of an operand is row r % 61 of a random
    block); checked: 8 rows x 8 columns of every 32nd group and of the last."""
    G = 257
    counts = np.concatenate([synth.gen_group_counts(131072, G - 1, seed=0), [16384]])
    offs = _offsets(counts)
    Mt = int(offs[-1])
    cap = M.wgrad_chunks(Mt, G)
    pref = OQ.chunk_prefix(offs)
    log(f"[wgrad full] N={N} K={K}: M={Mt} chunks {cap}")
    yb, ab = _codes((61, 128 * cap), 71), _codes((59, 128 * cap), 72)
    sY = synth.pow2_scales((N, cap), 73, -2, 2)
    sA = synth.pow2_scales((K, cap), 74, -2, 2)
    # chunk-major operands: [c, n, i] = yb[n % 61, 128 c + i]
    qY_d = torch.from_numpy(yb).cuda().view(61, cap, 128)[torch.arange(N, device="cuda") % 61]
    qY_d = qY_d.permute(1, 0, 2).contiguous()
    qA_d = torch.from_numpy(ab).cuda().view(59, cap, 128)[torch.arange(K, device="cuda") % 59]
    qA_d = qA_d.permute(1, 0, 2).contiguous()
    dW = torch.empty((G, N, K), dtype=torch.float32, device="cuda")
    log(f"[wgrad full] N={N} K={K}: launch")
    M.grouped_fp8_wgrad(qY_d, dev(np.ascontiguousarray(sY.T)), qA_d, dev(np.ascontiguousarray(sA.T)), cap,
                        dev(offs.astype(np.int32)), G, Mt, N, K, dW)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    for g in list(range(0, G, 32)) + [G - 1]:
        ns = np.sort(rng.choice(N, 8, replace=False))
        ks = np.sort(rng.choice(K, 8, replace=False))
        cs = slice(int(pref[g]) * 128, int(pref[g + 1]) * 128)
        ref = OG.grouped_wgrad(yb[ns % 61][:, cs], sY[ns][:, cs.start // 128:cs.stop // 128],
                               ab[ks % 59][:, cs], sA[ks][:, cs.start // 128:cs.stop // 128],
                               [0, int(pref[g + 1] - pref[g])])[0].astype(np.float32)
        got = host(dW[g][torch.from_numpy(ns).cuda()][:, torch.from_numpy(ks).cuda()])
        assert np.array_equal(got, ref), (g, int((got != ref).sum()))
    log(f"[wgrad full] N={N} K={K}: sampled entries bit-exact")
