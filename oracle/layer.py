"""The DeepSeekMoE layer forward, end to end (test infrastructure only).

Composition of the steps in this package, in the order the method applies
them: route (sigmoid + selection bias + group-limited top-k), quantise the
activations 1x128, dispatch (permute by expert), grouped gate+up GEMM,
SwiGLU + requantisation, grouped down GEMM, weighted combine plus shared
expert.  Storage points mirror the GPU path: bf16 after each GEMM and for the
output, E4M3 codes with fp32 1x128 scales for x and h (news.qq.com/rain/a/
20241229A05OQF00, section FP8 低精度训练 › 低精度存储和通信).

Two forms are given:

* ``layer``        - grouped form through the permutation (the shape of the
  GPU path);
* ``layer_tokens`` - direct per-token form: for each token, evaluate the
  chosen experts one by one and sum.  It shares the step functions but not
  the permutation / grouping / combine machinery, and it only needs the
  weights of the experts the given tokens touch (full-size sampled checks).
"""
from __future__ import annotations

from functools import lru_cache

import numpy as np

from .formats import bf16_value_from_bits, bf16_round
from .quant import quant_1x128, quant_128x128
from .route import route, router_scores, select
from .permute import permute
from .gemm import grouped_gemm, block_scaled_matmul, to_bf16
from .swiglu import swiglu_quant


class ExpertWeights:
    """Lazily quantised expert weights (128x128 blocks), cached per expert.

    ``fp32_gu(e)`` / ``fp32_dn(e)`` return fp32 [2I, H] and [H, I] arrays for
    expert e (e == E is the shared expert).
    """

    def __init__(self, fp32_gu, fp32_dn):
        self._gu = lru_cache(maxsize=None)(lambda e: quant_128x128(fp32_gu(e)))
        self._dn = lru_cache(maxsize=None)(lambda e: quant_128x128(fp32_dn(e)))

    def prefetch(self, experts, threads: int = 8):
        """Quantise the given experts' weights ahead of use, on a thread pool."""
        from concurrent.futures import ThreadPoolExecutor
        experts = sorted(set(int(e) for e in experts))
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda e: (self.gu(e), self.dn(e)), experts))

    def gu(self, e):
        return self._gu(e)

    def dn(self, e):
        return self._dn(e)


def layer(x_bits, centroids, bias, wts: ExpertWeights, n_group, topk_group, k, I,
          n_shared: int = 1, fused: bool = True):
    """fused=True: SwiGLU reads the gate/up sums in FP32 (never stored);
    fused=False: they are stored as bf16 first."""
    T, H = x_bits.shape
    E = centroids.shape[0]
    assert n_shared in (0, 1)
    r = route(x_bits, centroids, bias, n_group, topk_group, k)
    xv = bf16_value_from_bits(x_bits).astype(np.float32)
    xq, xs = quant_1x128(xv)
    offsets, perm_src, inv_perm = permute(r["idx"], E, n_shared)
    A, sA = xq[perm_src], xs[perm_src]
    G = E + n_shared
    gu = [wts.gu(g) for g in range(G)]
    dn = [wts.dn(g) for g in range(G)]
    Hgu = grouped_gemm(A, sA, [q for q, _ in gu], [s for _, s in gu], offsets)
    if not fused:
        Hgu = to_bf16(Hgu)
    Hq, Hs, h = swiglu_quant(Hgu, I)
    D = to_bf16(grouped_gemm(Hq, Hs, [q for q, _ in dn], [s for _, s in dn], offsets))
    shared = D[T * k:T * k + T] if n_shared else None
    from .combine import combine
    y, y64 = combine(D, inv_perm, r["w32"], T, k, shared)
    return dict(route=r, xq=xq, xs=xs, offsets=offsets, perm_src=perm_src,
                inv_perm=inv_perm, Hgu=Hgu, Hq=Hq, Hs=Hs, h=h, D=D, y=y, y64=y64)


def expert_ffn(xq_row, xs_row, wts: ExpertWeights, e: int, I: int, fused: bool = True,
               keep: bool = False):
    """One expert on quantised rows: gate+up GEMM, SwiGLU+requant, down GEMM.

    Returns the bf16 values of the down projection; with keep, also the
    exact gate/up sums (float64, before any rounding) as (D, hgu)."""
    qgu, sgu = wts.gu(e)
    qdn, sdn = wts.dn(e)
    hgu = block_scaled_matmul(xq_row, xs_row, qgu, sgu)
    exact = hgu
    if not fused:
        hgu = bf16_round(hgu)
    hq, hs, _ = swiglu_quant(hgu, I)
    D = bf16_round(block_scaled_matmul(hq, hs, qdn, sdn))
    return (D, exact) if keep else D


def layer_tokens(x_bits, centroids, bias, wts: ExpertWeights, n_group, topk_group, k, I,
                 tokens, n_shared: int = 1, fused: bool = True, keep: bool = False,
                 threads: int = 1):
    """Direct per-token form for the given token indices.

    Routing of a token only depends on that token (the counts are not an
    input of the forward), so the routes of a subset equal those of the full
    batch.  Each expert is evaluated on the sampled tokens that chose it (its
    rows are independent of one another), then every token's output is the
    sum over its slots in slot order plus the shared expert(s).
    Returns dict(idx, w32, margin, y (bf16 values), y64); with keep also
    hgu float64 [n, k + n_shared, 2I] (the exact gate/up sums of token i's
    slot j, shared expert(s) last) and D [n, k + n_shared, H] (bf16 values of
    the down projection).  threads > 1 evaluates the experts on a thread
    pool (the result does not depend on it).
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    E = centroids.shape[0]
    xs_bits = x_bits[tokens]
    s, sb = router_scores(xs_bits, centroids, bias)
    idx, w, margin = select(s, sb, n_group, topk_group, k)
    w32 = w.astype(np.float32)
    xq, xsc = quant_1x128(bf16_value_from_bits(xs_bits).astype(np.float32))
    n = len(tokens)
    H = x_bits.shape[1]

    def run(e):
        if e < E:
            rows, slots = np.nonzero(idx == e)
        else:
            rows = np.arange(n)
            slots = np.full(n, k + e - E)
        return rows, slots, expert_ffn(xq[rows], xsc[rows], wts, e, I, fused, keep=True)

    experts = sorted(set(idx.ravel().tolist())) + [E + sh for sh in range(n_shared)]
    if threads > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(threads) as ex:
            results = list(ex.map(run, experts))
    else:
        results = [run(e) for e in experts]
    D = np.zeros((n, k + n_shared, H), dtype=np.float64)
    hgu = np.zeros((n, k + n_shared, 2 * I), dtype=np.float64) if keep else None
    for rows, slots, (d, exact) in results:
        D[rows, slots] = d
        if keep:
            hgu[rows, slots] = exact
    y64 = np.zeros((n, H), dtype=np.float64)
    for i in range(n):
        for j in range(k):
            y64[i] += np.float64(w32[i, j]) * D[i, j]
        for sh in range(n_shared):
            y64[i] += D[i, k + sh]
    out = dict(idx=idx, w32=w32, margin=margin, y=bf16_round(y64), y64=y64)
    if keep:
        out.update(hgu=hgu, D=D, xq=xq, xs=xsc)
    return out
