"""Block-scaled FP8 grouped GEMM (test infrastructure only).

Operands are E4M3FN codes with fp32 scales: A per 1x128 tile, B per 128x128
block (news.qq.com/rain/a/20241229A05OQF00, section FP8 低精度训练 ›
细粒度量化).  Products are accumulated in high precision (same article,
提高累加精度, which keeps the MMA partials in FP32).  For every 128-wide K
block the partial dot product is taken exactly and multiplied by the product
of the two block scales; the oracle adds the blocks in float64.  With E4M3
operands each 128-term partial is exact in float64, so the result is the
exact value up to float64 rounding of the scaled sums.  The output is then
rounded once to bf16, the storage format of the GEMM outputs.

B is stored [G, N, K] (K contiguous), B's scales [G, N/128, K/128].
"""
from __future__ import annotations

import numpy as np

from .formats import e4m3_decode, bf16_round

TILE = 128


def block_scaled_matmul(qA, sA, qB, sB) -> np.ndarray:
    """One group: qA [m, K] codes, sA [m, K/128]; qB [N, K] codes, sB [N/128, K/128].

    C[i, n] = sum_kb sA[i, kb] * sB[n // 128, kb] * sum_{k in kb} A[i, k] B[n, k]
    """
    qA = np.asarray(qA)
    m, K = qA.shape
    N = qB.shape[0]
    nkb = K // TILE
    A = e4m3_decode(qA)
    B = e4m3_decode(qB)
    sA64 = np.asarray(sA, dtype=np.float32).astype(np.float64)
    sBn = np.repeat(np.asarray(sB, dtype=np.float32).astype(np.float64), TILE, axis=0)  # [N, nkb]
    C = np.zeros((m, N), dtype=np.float64)
    for kb in range(nkb):
        ks = slice(kb * TILE, (kb + 1) * TILE)
        part = A[:, ks] @ B[:, ks].T                       # exact
        C += (sA64[:, kb][:, None] * sBn[:, kb][None, :]) * part
    return C


def grouped_gemm(qA, sA, qB_groups, sB_groups, offsets) -> np.ndarray:
    """Grouped form: rows offsets[g]:offsets[g+1] of A use group g's B.

    qB_groups / sB_groups: indexable by group (array [G, N, K] or a list).
    Returns float64 [M_total, N] (not yet rounded).
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    G = len(offsets) - 1
    M = int(offsets[-1])
    N = qB_groups[0].shape[0]
    C = np.zeros((M, N), dtype=np.float64)
    for g in range(G):
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        if r1 > r0:
            C[r0:r1] = block_scaled_matmul(qA[r0:r1], sA[r0:r1], qB_groups[g], sB_groups[g])
    return C


def to_bf16(C: np.ndarray) -> np.ndarray:
    """Storage rounding of GEMM outputs (bf16, ties to even), as float64 values."""
    return bf16_round(C)


# ---- input gradient (backward for input) of the expert GEMMs -------------
#
# The forward product of a group is C = A W^T (C[i, n] = sum_k A[i, k] W[n, k]),
# so the gradient with respect to A of a loss with gradient dY = dL/dC is
# dA = dY W, a contraction over n.  In FP8 (news.qq.com article, section FP8
# 低精度训练: FP8 compute with 1x128 activation tiles and 128x128 weight
# blocks; the pipeline figure of the same article names the "backward for
# input" chunks) dY is quantised in 1x128 tiles along n, its contraction
# axis, and W keeps its 128x128 blocks.


def transpose_blocks(qW, sW):
    """Weights [..., N, K] with scales [..., N/128, K/128] -> W^T [..., K, N] with
    scales [..., K/128, N/128].  A 128x128 block's codes move as they are and its
    one scale moves with it, so the result quantises W^T exactly."""
    qW = np.asarray(qW)
    sW = np.asarray(sW)
    return np.ascontiguousarray(np.swapaxes(qW, -1, -2)), np.ascontiguousarray(np.swapaxes(sW, -1, -2))


def block_scaled_dgrad(qdY, sdY, qW, sW) -> np.ndarray:
    """One group: qdY [m, N] codes with 1x128 scales sdY [m, N/128]; qW [N, K] codes
    with 128x128 scales sW [N/128, K/128].

    dA[i, k] = sum_nb sdY[i, nb] * sW[nb, k // 128] * sum_{n in nb} dY[i, n] W[n, k]
    (each 128-term partial exact in float64, blocks added in float64).
    """
    qdY = np.asarray(qdY)
    m, N = qdY.shape
    K = np.asarray(qW).shape[1]
    dY = e4m3_decode(qdY)
    W = e4m3_decode(qW)
    sY = np.asarray(sdY, dtype=np.float32).astype(np.float64)
    sWk = np.repeat(np.asarray(sW, dtype=np.float32).astype(np.float64), TILE, axis=1)  # [N/128, K]
    dA = np.zeros((m, K), dtype=np.float64)
    for nb in range(N // TILE):
        ns = slice(nb * TILE, (nb + 1) * TILE)
        part = dY[:, ns] @ W[ns, :]                        # exact
        dA += (sY[:, nb][:, None] * sWk[nb][None, :]) * part
    return dA


def grouped_dgrad(qdY, sdY, qW_groups, sW_groups, offsets) -> np.ndarray:
    """Rows offsets[g]:offsets[g+1] of dY use group g's W.  float64 [M_total, K]."""
    offsets = np.asarray(offsets, dtype=np.int64)
    G = len(offsets) - 1
    M = int(offsets[-1])
    K = np.asarray(qW_groups[0]).shape[1]
    dA = np.zeros((M, K), dtype=np.float64)
    for g in range(G):
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        if r1 > r0:
            dA[r0:r1] = block_scaled_dgrad(qdY[r0:r1], sdY[r0:r1], qW_groups[g], sW_groups[g])
    return dA


# ---- weight gradient (backward for weights) of the expert GEMMs ----------
#
# For group g the forward C_g = A_g W_g^T has dW_g = dY_g^T A_g, a
# contraction over the group's tokens.  Both operands come quantised in
# 128x1 tiles along the tokens (quant.quant_128x1_grouped: transposed, each
# group padded to whole 128-token chunks), so each 128-token chunk is one
# partial with one scale per (output row, chunk) on either side.


def grouped_wgrad(qYT, sYT, qAT, sAT, chunk_pref) -> np.ndarray:
    """qYT [N, P] codes, sYT [N, P/128]; qAT [K, P], sAT [K, P/128]; group g owns
    chunks [chunk_pref[g], chunk_pref[g+1]).  Returns float64 [G, N, K]:

    dW[g, n, k] = sum_{c in g} sYT[n, c] * sAT[k, c] * sum_{j<128} Y[n, 128c+j] A[k, 128c+j]
    (exact 128-term partials, chunks added in float64 in order).
    """
    chunk_pref = np.asarray(chunk_pref, dtype=np.int64)
    G = len(chunk_pref) - 1
    Y = e4m3_decode(qYT)
    A = e4m3_decode(qAT)
    sY = np.asarray(sYT, dtype=np.float32).astype(np.float64)
    sA = np.asarray(sAT, dtype=np.float32).astype(np.float64)
    N, K = Y.shape[0], A.shape[0]
    dW = np.zeros((G, N, K), dtype=np.float64)
    for g in range(G):
        for c in range(int(chunk_pref[g]), int(chunk_pref[g + 1])):
            cs = slice(c * TILE, (c + 1) * TILE)
            part = Y[:, cs] @ A[:, cs].T                   # exact
            dW[g] += (sY[:, c][:, None] * sA[:, c][None, :]) * part
    return dW
