"""SwiGLU and requantisation of the expert hidden state (test infrastructure only).

The pages do not name the expert FFN form; the workload defines it as SwiGLU
with a fused gate+up projection: columns [0, I) of the first GEMM are the gate
g, columns [I, 2I) the up projection u, and h = silu(g) * u with
silu(g) = g / (1 + exp(-g)).  h is then quantised in 1x128 tiles like any
activation (news.qq.com/rain/a/20241229A05OQF00, section FP8 低精度训练 ›
细粒度量化, and 低精度存储和通信 for keeping activations in FP8).

Two readings of where g and u come from are supported:
* unfused - the first GEMM stores bf16 g and u, which SwiGLU reads back;
* fused   - g and u are never stored: SwiGLU reads the first GEMM's FP32
  totals (the pages keep MMA results in FP32 and store activations in FP8 or
  BF16 only; g and u are not stored at all in this form).  The oracle takes
  the fp32 rounding of the exact sums.
Either way h decides E4M3 codes, so it is evaluated in fp32, the kernel's
precision, in this order: t = exp(-g); d = 1 + t; a = g / d; h = a * u.
"""
from __future__ import annotations

import numpy as np

from .quant import quant_1x128


def silu_mul_fp32(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    g = np.asarray(g, dtype=np.float32)
    u = np.asarray(u, dtype=np.float32)
    t = np.exp(-g).astype(np.float32)
    d = (np.float32(1.0) + t).astype(np.float32)
    a = (g / d).astype(np.float32)
    return (a * u).astype(np.float32)


def swiglu_quant(hgu: np.ndarray, I: int):
    """hgu [M, 2I]: bf16 values (unfused) or exact float64 sums (fused; rounded
    to fp32 here, ties to even).  Returns (codes uint8 [M, I], scales fp32
    [M, I/128], h fp32)."""
    hgu = np.asarray(hgu, dtype=np.float64)
    g = hgu[:, :I].astype(np.float32)
    u = hgu[:, I:2 * I].astype(np.float32)
    h = silu_mul_fp32(g, u)
    q, s = quant_1x128(h)
    return q, s, h
