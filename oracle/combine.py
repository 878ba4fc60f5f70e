"""Weighted combine plus shared expert (test infrastructure only).

Each token's output is the gate-weighted sum of its routed experts' outputs
plus the shared expert's output, unweighted (DeepSeekMoE with one shared and
256 routed experts: news.qq.com/rain/a/20241229A05OQF00, section
DeepSeekMoE 架构; the all-to-all combine of section DualPipe 流水线并行 is
this gather on one GPU).  Summed in float64, then rounded once to bf16.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_round


def combine(D: np.ndarray, inv_perm: np.ndarray, w: np.ndarray, T: int, k: int,
            shared: np.ndarray | None):
    """D: bf16-valued [R, H]; inv_perm [T*k]; w fp32 [T, k]; shared [T, H] or None.

    Returns (y_bf16 float64 [T, H], y64 float64 [T, H]).
    """
    D = np.asarray(D, dtype=np.float64)
    w64 = np.asarray(w, dtype=np.float32).astype(np.float64).reshape(T, k)
    rows = np.asarray(inv_perm, dtype=np.int64).reshape(T, k)
    y = np.zeros((T, D.shape[1]), dtype=np.float64)
    for j in range(k):
        y += w64[:, j][:, None] * D[rows[:, j]]
    if shared is not None:
        y += np.asarray(shared, dtype=np.float64)
    return bf16_round(y), y
