"""Aux-loss-free bias update (test infrastructure only).

The per-expert selection bias is lowered for experts that carried more than
their share of the batch and raised for experts that carried less; no loss
term is involved: aliyun study note (developer.aliyun.com/article/1776647),
section 2.2; news.qq.com/rain/a/20241229A05OQF00, section 无额外损耗的负载均衡,
which gives the update speed gamma = 0.001 for the first 14.3T tokens (0.0
after).  Reading: "load" is the count of assignments in this batch, "share"
is the mean T*k/E, a count equal to the mean leaves the bias unchanged.  The
update is done in fp32, the precision of the stored bias.

Sequence-wise balance statistic: the news.qq.com article (section
无额外损耗的负载均衡) sets its factor alpha = 0.0001, and the V3 summary at
m.jxzklqfsx.com/aigc/3586.html (section （二）無輔助損失負載均衡策略革新) has it
complement the bias by guarding against imbalance inside one sequence; no
page prints the formula.  Reading (the usual form of such a balance term,
stated on its own terms): for a sequence of L consecutive tokens, with s the
unbiased sigmoid scores of all E routed experts and s' = s / sum_e s per token,
    P_e = (1/L) sum_t s'_{t,e},   f_e = E / (k L) * #{t : e chosen for t},
    L_bal = alpha * sum_e f_e P_e.
f is piecewise constant (it counts the selection), so only P carries a
gradient.  Sequences are consecutive runs of seq_len tokens; the last may be
shorter.
"""
from __future__ import annotations

import numpy as np

GAMMA = 0.001
ALPHA = 0.0001


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


def seq_bounds(T: int, seq_len: int):
    """[(t0, t1)] of each sequence: consecutive runs of seq_len tokens."""
    return [(t0, min(T, t0 + seq_len)) for t0 in range(0, T, seq_len)]


def seq_balance(s, idx, seq_len: int, alpha: float = ALPHA):
    """s float64 [T, E] (unbiased scores of every routed expert), idx [T, k]
    (the chosen experts).  Returns dict(f, P float64 [B, E], loss float64 [B])."""
    s = np.asarray(s, dtype=np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    T, E = s.shape
    k = idx.shape[1]
    sn = s / s.sum(axis=1, keepdims=True)
    bounds = seq_bounds(T, seq_len)
    f = np.zeros((len(bounds), E))
    P = np.zeros((len(bounds), E))
    for b, (t0, t1) in enumerate(bounds):
        L = t1 - t0
        f[b] = E * np.bincount(idx[t0:t1].reshape(-1), minlength=E) / (k * L)
        P[b] = sn[t0:t1].sum(axis=0) / L
    return dict(f=f, P=P, loss=alpha * np.sum(f * P, axis=1))


def seq_balance_grad_logits(s, idx, seq_len: int, alpha: float = ALPHA):
    """Gradient of the sum over sequences of L_bal with respect to the router
    logits (s = sigmoid(logit)), the selection held fixed: float64 [T, E].
    With S = sum_e s:  dL/ds_e = (alpha / L) (f_e - sum_i f_i s'_i) / S, then
    times s_e (1 - s_e)."""
    s = np.asarray(s, dtype=np.float64)
    st = seq_balance(s, idx, seq_len, alpha)
    T, E = s.shape
    S = s.sum(axis=1, keepdims=True)
    sn = s / S
    g = np.zeros_like(s)
    for b, (t0, t1) in enumerate(seq_bounds(T, seq_len)):
        fb = st["f"][b][None, :]
        ds = alpha / (t1 - t0) * (fb - np.sum(fb * sn[t0:t1], axis=1, keepdims=True)) / S[t0:t1]
        g[t0:t1] = ds * s[t0:t1] * (1.0 - s[t0:t1])
    return g
