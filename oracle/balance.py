"""Aux-loss-free bias update (test infrastructure only).

The per-expert selection bias is lowered for experts that carried more than
their share of the batch and raised for experts that carried less; no loss
term is involved: aliyun study note (developer.aliyun.com/article/1776647),
section 2.2; news.qq.com/rain/a/20241229A05OQF00, section 无额外损耗的负载均衡,
which gives the update speed gamma = 0.001 for the first 14.3T tokens (0.0
after).  Reading: "load" is the count of assignments in this batch, "share"
is the mean T*k/E, a count equal to the mean leaves the bias unchanged.  The
update is done in fp32, the precision of the stored bias.
"""
from __future__ import annotations

import numpy as np

GAMMA = 0.001


def bias_update(counts: np.ndarray, bias: np.ndarray, gamma: float = GAMMA) -> np.ndarray:
    counts = np.asarray(counts, dtype=np.int64)
    b = np.asarray(bias, dtype=np.float32).copy()
    E = counts.shape[0]
    total = int(counts.sum())
    g = np.float32(gamma)
    over = counts * E > total      # c_e > mean, compared exactly in integers
    under = counts * E < total
    b[over] = b[over] - g
    b[under] = b[under] + g
    return b.astype(np.float32)
