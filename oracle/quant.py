"""Fine-grained FP8 quantisation (test infrastructure only).

Activations are scaled per 1x128 tile (one row, 128 consecutive columns) and
weights per 128x128 block: news.qq.com/rain/a/20241229A05OQF00, section
FP8 低精度训练 › 细粒度量化; the aliyun study note (developer.aliyun.com/
article/1776647) section 4.1 names the 128x128 weight blocks.

The pages do not give the scale rule.  Reading used here (the same for both
granularities): the scale is s = amax / 448 computed in fp32, or 1 when the
tile is all zero; each element is divided by s (one correctly rounded fp32
division) and encoded to E4M3FN with round-to-nearest-even and saturation.
The code decision is taken in fp32 because that is the kernel's precision.
"""
from __future__ import annotations

import numpy as np

from .formats import e4m3_encode, e4m3_decode

TILE = 128
FP8_MAX = np.float32(448.0)


def _scale_from_amax(amax: np.ndarray) -> np.ndarray:
    amax = np.asarray(amax, dtype=np.float32)
    s = np.where(amax > 0, amax / FP8_MAX, np.float32(1.0))
    return s.astype(np.float32)


def quant_1x128(v: np.ndarray):
    """Quantise values v [M, K] (K % 128 == 0) in 1x128 tiles.

    Returns codes uint8 [M, K] and scales fp32 [M, K/128] (row-major).
    v must be exactly representable in fp32 (bf16 inputs, fp32 SwiGLU).
    """
    v = np.asarray(v, dtype=np.float32)
    M, K = v.shape
    assert K % TILE == 0, K
    t = v.reshape(M, K // TILE, TILE)
    amax = np.abs(t).max(axis=2)
    s = _scale_from_amax(amax)
    scaled = (t / s[:, :, None]).astype(np.float32)  # fp32 division, RNE
    q = e4m3_encode(scaled).reshape(M, K)
    return q, s


def quant_128x128(w: np.ndarray):
    """Quantise a weight matrix w [N, K] (both % 128 == 0) in 128x128 blocks.

    Returns codes uint8 [N, K] and scales fp32 [N/128, K/128].
    """
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    assert N % TILE == 0 and K % TILE == 0, (N, K)
    b = w.reshape(N // TILE, TILE, K // TILE, TILE)
    amax = np.abs(b).max(axis=(1, 3))
    s = _scale_from_amax(amax)
    scaled = (b / s[:, None, :, None]).astype(np.float32)
    q = e4m3_encode(scaled).reshape(N, K)
    return q, s


def dequant_1x128(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    M, K = q.shape
    return (e4m3_decode(q).reshape(M, K // TILE, TILE)
            * s.astype(np.float64)[:, :, None]).reshape(M, K)


def dequant_128x128(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    N, K = q.shape
    return (e4m3_decode(q).reshape(N // TILE, TILE, K // TILE, TILE)
            * s.astype(np.float64)[:, None, :, None]).reshape(N, K)


def chunk_prefix(offsets) -> np.ndarray:
    """Exclusive prefix over groups of ceil(rows / 128): group g's token chunks
    are [pref[g], pref[g+1]) in a layout that pads every group to whole
    128-token chunks."""
    offsets = np.asarray(offsets, dtype=np.int64)
    rows = np.diff(offsets)
    return np.concatenate([[0], np.cumsum((rows + TILE - 1) // TILE)]).astype(np.int64)


def quant_128x1_grouped(v: np.ndarray, offsets):
    """Quantise v [M, C] in 128x1 tiles along the token axis, per group.

    The weight gradient of an expert contracts over that expert's tokens, so
    its FP8 operands need one scale per 128 tokens of one column (the 1x128
    tile of the transposed matrix; the pages give 1x128 activation tiles
    without the backward orientation - this is the reading used).  Group g
    (rows offsets[g]:offsets[g+1]) is cut into 128-row chunks from its first
    row; a last partial chunk is padded with zeros.

    Returns codes uint8 [C, P] and scales fp32 [C, P/128], transposed (tokens
    contiguous), P = 128 * chunk_prefix(offsets)[-1]: column 128*c + j of the
    output is row j of chunk c.  Padding codes are 0; an all-zero tile has
    scale 1.
    """
    v = np.asarray(v, dtype=np.float32)
    M, C = v.shape
    pref = chunk_prefix(offsets)
    offsets = np.asarray(offsets, dtype=np.int64)
    P = int(pref[-1]) * TILE
    padded = np.zeros((P, C), dtype=np.float32)
    for g in range(len(offsets) - 1):
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        p0 = int(pref[g]) * TILE
        padded[p0:p0 + (r1 - r0)] = v[r0:r1]
    q, s = quant_1x128(np.ascontiguousarray(padded.T))
    return q, s
