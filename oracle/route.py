"""Router: sigmoid scores, selection bias, group-limited top-k (test infrastructure only).

Follows, in order:

* scores are sigmoid gates of the token-centroid affinity - aliyun study
  note (developer.aliyun.com/article/1776647), section 2.2 (V3 的做法：
  偏置项动态调节);
* every expert carries a bias that is added to its score for the top-k
  choice only; the gate weights use the unbiased scores - same section, and
  the news.qq.com article (news.qq.com/rain/a/20241229A05OQF00), section
  无额外损耗的负载均衡;
* each token picks 8 of 256 routed experts and reaches at most 4 nodes -
  news.qq.com article, sections DeepSeekMoE 架构 and 通信优化 › 节点限制路由.

Readings where the pages are silent (listed in the design notes): nodes are
contiguous groups of E/n_group experts; a group's score is the sum of its two
largest biased scores; the topk_group best groups are kept; among the kept
experts the k largest biased scores are chosen; ties go to the lower index;
the chosen ids are emitted in ascending order; the weights are the unbiased
scores of the chosen experts divided by their sum.

Precision: the pages keep gating in high precision (news.qq.com article,
section FP8 低精度训练 › 选择性高精度).  The oracle computes everything in
float64 and reports, per token, the margin that decides the selection.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_value_from_bits


def router_scores(x_bits: np.ndarray, centroids: np.ndarray, bias: np.ndarray):
    """Return (s, s_biased) in float64, each [T, E]."""
    x = bf16_value_from_bits(x_bits)                    # exact widening
    c = np.asarray(centroids, dtype=np.float32).astype(np.float64)
    logits = x @ c.T                                     # float64 matmul
    s = 1.0 / (1.0 + np.exp(-logits))
    sb = s + np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :]
    return s, sb


def select(s: np.ndarray, sb: np.ndarray, n_group: int, topk_group: int, k: int):
    """Group-limited top-k on biased scores sb; weights from unbiased s.

    Returns idx int32 [T, k] (ascending expert id), w float64 [T, k],
    margin float64 [T] (smallest gap that decided the selection; inf when the
    choice is forced).
    """
    T, E = s.shape
    assert E % n_group == 0
    gs = E // n_group
    assert gs >= 2 and 1 <= topk_group <= n_group and 1 <= k <= topk_group * gs

    grouped = sb.reshape(T, n_group, gs)
    two = -np.sort(-grouped, axis=2)[:, :, :2]
    gscore = two[:, :, 0] + two[:, :, 1]                # [T, n_group]

    # stable sort on -score: equal scores keep ascending group index
    gorder = np.argsort(-gscore, axis=1, kind="stable")
    kept = gorder[:, :topk_group]
    gmask = np.zeros((T, n_group), dtype=bool)
    np.put_along_axis(gmask, kept, True, axis=1)
    emask = np.repeat(gmask, gs, axis=1)

    cand = np.where(emask, sb, -np.inf)
    eorder = np.argsort(-cand, axis=1, kind="stable")
    chosen = np.sort(eorder[:, :k], axis=1)
    idx = chosen.astype(np.int32)

    ssel = np.take_along_axis(s, chosen, axis=1)
    w = ssel / ssel.sum(axis=1, keepdims=True)

    gs_sorted = np.take_along_axis(gscore, gorder, axis=1)
    if topk_group < n_group:
        gmargin = gs_sorted[:, topk_group - 1] - gs_sorted[:, topk_group]
    else:
        gmargin = np.full(T, np.inf)
    c_sorted = np.take_along_axis(cand, eorder, axis=1)
    if k < topk_group * gs:
        emargin = c_sorted[:, k - 1] - c_sorted[:, k]
    else:
        emargin = np.full(T, np.inf)
    margin = np.minimum(gmargin, emargin)
    return idx, w, margin


def route(x_bits, centroids, bias, n_group: int, topk_group: int, k: int):
    """Full router: returns dict(idx, w (float64), w32, counts, margin, s, sb)."""
    s, sb = router_scores(x_bits, centroids, bias)
    idx, w, margin = select(s, sb, n_group, topk_group, k)
    E = s.shape[1]
    counts = np.bincount(idx.ravel(), minlength=E).astype(np.int32)
    return dict(idx=idx, w=w, w32=w.astype(np.float32), counts=counts,
                margin=margin, s=s, sb=sb)
