"""Dispatch order: tokens permuted by expert (test infrastructure only).

The pages split each chunk into attention, all-to-all dispatch, MLP and
all-to-all combine (news.qq.com/rain/a/20241229A05OQF00, section DualPipe
流水线并行).  On one GPU the dispatch is a permutation of the token-expert
assignments into expert-contiguous rows.  Reading: rows of expert e appear in
ascending (token, slot) order; the n_shared shared expert(s) follow as one
block of T rows each, in token order.
"""
from __future__ import annotations

import numpy as np


def permute(idx: np.ndarray, E: int, n_shared: int = 1):
    """idx int [T, k] -> (offsets [E+n_shared+1], perm_src [T*k+n_shared*T],
    inv_perm [T*k]).

    offsets: exclusive prefix sum of the group sizes (counts..., T per shared).
    perm_src[r]: token whose row is r.  inv_perm[t*k+j]: row of (t, j).
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    flat = idx.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=E)
    sizes = np.concatenate([counts, np.full(n_shared, T, dtype=np.int64)])
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    order = np.argsort(flat, kind="stable")       # expert-major, (t, j) ascending
    perm_src = np.empty(T * k + n_shared * T, dtype=np.int32)
    perm_src[: T * k] = order // k
    for s in range(n_shared):
        perm_src[T * k + s * T: T * k + (s + 1) * T] = np.arange(T)
    inv_perm = np.empty(T * k, dtype=np.int32)
    inv_perm[order] = np.arange(T * k, dtype=np.int32)
    return offsets, perm_src, inv_perm
