"""Pins of the oracle's block-scaled grouped GEMM: exact integer cases against
a pure-Python loop, dequantise-then-matmul for one group, scale-block
indexing with a non-square, non-symmetric layout, and group boundaries."""
import numpy as np
import pytest

import synth
from oracle import formats as F
from oracle import gemm as GM
from oracle import quant as Q


def _int_codes(shape, seed):
    v = synth.int_fp8_operand(shape, seed)
    return F.e4m3_encode(v), v


def test_integer_case_matches_python_loop():
    M, N, K = 5, 256, 256
    qA, A = _int_codes((M, K), 1)
    qB, B = _int_codes((N, K), 2)
    sA = synth.pow2_scales((M, K // 128), 3)
    sB = synth.pow2_scales((N // 128, K // 128), 4)
    C = GM.block_scaled_matmul(qA, sA, qB, sB)
    for i in range(M):
        for n in range(0, N, 37):
            acc = 0.0
            for k in range(K):
                acc += float(A[i, k]) * float(B[n, k]) * float(sA[i, k // 128]) * float(sB[n // 128, k // 128])
            assert C[i, n] == acc


def test_one_group_equals_dequantised_matmul():
    rng = np.random.default_rng(0)
    a = rng.standard_normal((40, 384)).astype(np.float32)
    w = (rng.standard_normal((256, 384)) * 0.02).astype(np.float32)
    qA, sA = Q.quant_1x128(a)
    qB, sB = Q.quant_128x128(w)
    C = GM.block_scaled_matmul(qA, sA, qB, sB)
    ref = Q.dequant_1x128(qA, sA) @ Q.dequant_128x128(qB, sB).T
    np.testing.assert_allclose(C, ref, rtol=1e-12, atol=1e-12)
    # transposed operands or swapped scale axes would not match
    assert not np.allclose(C, Q.dequant_1x128(qA, sA) @ Q.dequant_128x128(qB, sB.T.copy().reshape(sB.shape)).T, rtol=1e-6) or sB.shape[0] == sB.shape[1]


def test_scale_blocks_are_indexed_by_n_and_k():
    M, N, K = 3, 384, 256          # 3 N-blocks x 2 K-blocks
    qA, A = _int_codes((M, K), 5)
    qB, B = _int_codes((N, K), 6)
    sA = np.ones((M, 2), np.float32)
    for nb in range(3):
        for kb in range(2):
            sB = np.ones((3, 2), np.float32)
            sB[nb, kb] = 8.0
            C = GM.block_scaled_matmul(qA, sA, qB, sB)
            base = A @ B.T
            extra = 7.0 * (A[:, kb * 128:(kb + 1) * 128] @ B[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128].T)
            exp = base.copy()
            exp[:, nb * 128:(nb + 1) * 128] += extra
            assert np.array_equal(C, exp)


def test_grouped_boundaries():
    G, N, K = 4, 128, 256
    offsets = np.array([0, 3, 3, 10, 12])         # one empty group
    qA, A = _int_codes((12, K), 7)
    sA = synth.pow2_scales((12, 2), 8)
    qB = np.stack([_int_codes((N, K), 10 + g)[0] for g in range(G)])
    sB = np.stack([synth.pow2_scales((1, 2), 20 + g) for g in range(G)])
    C = GM.grouped_gemm(qA, sA, qB, sB, offsets)
    for g in range(G):
        r0, r1 = offsets[g], offsets[g + 1]
        if r1 > r0:
            assert np.array_equal(C[r0:r1], GM.block_scaled_matmul(qA[r0:r1], sA[r0:r1], qB[g], sB[g]))
    # row 5 (group 2) computed with the wrong group would differ
    assert not np.array_equal(C[5:6], GM.block_scaled_matmul(qA[5:6], sA[5:6], qB[1], sB[1]))


def test_to_bf16_is_single_rounding():
    C = np.array([1.0 + 2.0 ** -8 + 2.0 ** -40, 1.0 + 2.0 ** -8, -3.0])
    assert GM.to_bf16(C).tolist() == [1.0 + 2.0 ** -7, 1.0, -3.0]
