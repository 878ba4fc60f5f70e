"""Standalone grouped GEMM at the full workload shape, through the C ABI.

256 groups, rows per group Multinomial(65536, uniform) at seed 0 (the counts
the benchmark times), no row gather, bf16 output; fused gate+up (K=7168,
N=4096) and down (K=2048, N=7168).

Operands are integer-valued E4M3 codes in [-2, 2] with power-of-two block
scales 2^[-2, 2] (news.qq.com article, section FP8 低精度训练 › 细粒度量化:
1x128 activation tiles, 128x128 weight blocks).  Every product, 128-term
block partial (|.| <= 512), scaled block and running sum (|.| < 2^19 on a
2^-4 grid) is exact in fp32, so the GPU's bf16 output must equal the
oracle's bf16 rounding of the exact result bit for bit.  The oracle computes
sampled rows only: the first, middle and last row of every 16th group and of
the last group.  Each group's B is a rotation of one random block, so the
test draws 29 MB of codes instead of 7.5 GB.
"""
import numpy as np
import pytest
import torch

import synth
import fp8_block_scaled_bias_amd as M
from gpu_common import bf16_values_host, log
from oracle import formats as OF
from oracle import gemm as OG

pytestmark = pytest.mark.gpu

G, ROWS = 256, 65536
VALS = np.arange(-2, 3, dtype=np.float32)


def _codes(shape, seed):
    lut = OF.e4m3_encode(VALS)
    v = synth.int_fp8_operand(shape, seed, -2, 2)
    return lut[(v + 2).astype(np.int8)]


def _group_b(base, g):
    return np.roll(base.ravel(), 7919 * g).reshape(base.shape)


@pytest.mark.parametrize("K,N", [(7168, 4096), (2048, 7168)], ids=["gate_up", "down"])
def test_grouped_gemm_full_shape_exact(K, N):
    counts = synth.gen_group_counts(ROWS, G, seed=0)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    log(f"[c5] K={K} N={N}: rows/group {counts.min()}..{counts.max()}")
    qA = _codes((ROWS, K), 11 + K)
    sA = synth.pow2_scales((ROWS, K // 128), 12 + K, -2, 2)
    base = _codes((N, K), 13 + K)
    sB = synth.pow2_scales((G, N // 128, K // 128), 14 + K, -2, 2)

    dev = "cuda"
    A_d = torch.from_numpy(qA).to(dev)
    sA_d = torch.from_numpy(sA).to(dev)
    base_d = torch.from_numpy(base).to(dev).flatten()
    B_d = torch.empty((G, N, K), dtype=torch.uint8, device=dev)
    for g in range(G):   # torch.roll matches np.roll (the oracle's _group_b)
        B_d[g].copy_(torch.roll(base_d, 7919 * g).view(N, K))
    sB_d = torch.from_numpy(sB).to(dev)
    offs_d = torch.from_numpy(offsets.astype(np.int32)).to(dev)
    C_d = torch.empty((ROWS, N), dtype=torch.bfloat16, device=dev)
    log(f"[c5] K={K} N={N}: launch")
    M.grouped_fp8_gemm(A_d, sA_d, None, B_d, sB_d, offs_d, G, ROWS, N, K, C_d)
    torch.cuda.synchronize()

    checked = 0
    for g in list(range(0, G, 16)) + [G - 1]:
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        rows = sorted({r0, (r0 + r1) // 2, r1 - 1})
        got = bf16_values_host(C_d[rows])
        ref = OG.to_bf16(OG.block_scaled_matmul(qA[rows], sA[rows], _group_b(base, g), sB[g]))
        assert np.array_equal(got, ref), (g, int((got != ref).sum()))
        checked += len(rows)
    log(f"[c5] K={K} N={N}: {checked} sampled rows bit-exact")
