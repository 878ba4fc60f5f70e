"""Backward of the DeepSeekMoE layer's expert path in FP8 (test infrastructure only).

The pages train the model in FP8 - 1x128 activation tiles, 128x128 weight
blocks, FP32 accumulation (news.qq.com/rain/a/20241229A05OQF00, section FP8
低精度训练) - and split each chunk's backward into backward-for-input and
backward-for-weights parts (section 工程 › DualPipe 流水线并行).  They give no
kernel-level recipe; the reading used here (the GPU path's):

* combine backward: the gate-weighted sum y = sum_j w_j D_r(j) + D_shared
  gives dD_r(j) = w_j dy, dD_shared = dy and dw_j = <dy, D_r(j)>; dD is
  stored as bf16 of the fp32 product w_j * dy (the kernel's precision);
* down: dh = dD W_dn (dgrad on 1x128-quantised dD), dW_dn = dD^T h (wgrad on
  128x1-quantised operands);
* SwiGLU backward from the bf16 gate/up outputs of the gate+up GEMM, which
  the backward recomputes (the fused forward keeps no g, u): with
  s = sigma(g), dg = dh u s (1 + g (1 - s)), du = dh g s, and h = g s u for
  the down wgrad; all stored as bf16;
* gate+up: dX = dGU W_gu on the permuted rows, dW_gu = dGU^T X;
* dx = sum over a token's rows of dX (the combine with unit weights).

Storage points mirror the GPU: bf16 after every elementwise step and GEMM,
E4M3 with fp32 scales for GEMM operands, FP32 weight gradients.  The router's
backward (router_backward, below) takes the gate weights' gradient dw to the
router's part of dx and to the centroids' gradient; layer_backward adds the
two parts of dx (one bf16 rounding of their sum, as the GPU stores it).
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_round, bf16_value_from_bits
from .gemm import grouped_dgrad, grouped_gemm, grouped_wgrad, to_bf16, transpose_blocks  # noqa: F401
from .quant import chunk_prefix, quant_1x128, quant_128x1_grouped


def combine_backward(dy, D, inv_perm, w, T: int, k: int, n_shared: int):
    """dy [T, H] and D [R, H] (bf16 values), inv_perm [T*k], w fp32 [T, k].

    Returns dict: dD64 (exact products), dD (bf16 of the fp32 products, the
    stored form), dw (float64 [T, k]).
    """
    dy = np.asarray(dy, dtype=np.float64)
    D = np.asarray(D, dtype=np.float64)
    w32 = np.asarray(w, dtype=np.float32).reshape(T, k)
    rows = np.asarray(inv_perm, dtype=np.int64).reshape(T, k)
    R, H = D.shape
    dD64 = np.zeros((R, H), dtype=np.float64)
    dD32 = np.zeros((R, H), dtype=np.float32)
    dw = np.zeros((T, k), dtype=np.float64)
    for j in range(k):
        dD64[rows[:, j]] = w32[:, j].astype(np.float64)[:, None] * dy
        dD32[rows[:, j]] = w32[:, j][:, None] * dy.astype(np.float32)
        dw[:, j] = np.sum(dy * D[rows[:, j]], axis=1)
    if n_shared:
        dD64[T * k:T * k + T] = dy
        dD32[T * k:T * k + T] = dy.astype(np.float32)
    return dict(dD64=dD64, dD=bf16_round(dD32.astype(np.float64)), dw=dw)


def swiglu_backward(gu, dh, I: int):
    """gu [M, 2I] = [g | u] and dh [M, I] (bf16 values).  float64:
    returns (dgu [M, 2I] = [dg | du], h [M, I])."""
    gu = np.asarray(gu, dtype=np.float64)
    dh = np.asarray(dh, dtype=np.float64)
    g, u = gu[:, :I], gu[:, I:2 * I]
    s = 1.0 / (1.0 + np.exp(-g))
    dg = dh * u * s * (1.0 + g * (1.0 - s))
    du = dh * g * s
    return np.concatenate([dg, du], axis=1), g * s * u


def expert_backward(dy_bits, fwd: dict, wts, x_bits, T: int, k: int, I: int, n_shared: int = 1):
    """Backward of the expert path of oracle.layer.layer's forward `fwd`
    (its route, permutation, quantised x and D) for the output gradient dy
    (bf16 bits [T, H]).  Returns dict with dx (bf16 values [T, H]), dw
    [T, k], dW_gu [G, 2I, H] and dW_dn [G, H, I] (float64 of the FP32
    results) and the intermediate stored tensors."""
    dy = bf16_value_from_bits(dy_bits)
    x = bf16_value_from_bits(x_bits)
    offsets = np.asarray(fwd["offsets"], dtype=np.int64)
    perm_src, inv_perm = fwd["perm_src"], fwd["inv_perm"]
    G = len(offsets) - 1
    gu = [wts.gu(g) for g in range(G)]
    dn = [wts.dn(g) for g in range(G)]
    cb = combine_backward(dy, fwd["D"], inv_perm, fwd["route"]["w32"], T, k, n_shared)
    dD = cb["dD"]
    q, s = quant_1x128(dD)
    dh = to_bf16(grouped_dgrad(q, s, [w for w, _ in dn], [sc for _, sc in dn], offsets))
    GU = to_bf16(grouped_gemm(fwd["xq"][perm_src], fwd["xs"][perm_src], [w for w, _ in gu],
                              [sc for _, sc in gu], offsets))
    dgu64, h64 = swiglu_backward(GU, dh, I)
    dGU, h = bf16_round(dgu64), bf16_round(h64)
    q, s = quant_1x128(dGU)
    dXp = to_bf16(grouped_dgrad(q, s, [w for w, _ in gu], [sc for _, sc in gu], offsets))
    rows = np.asarray(inv_perm, dtype=np.int64).reshape(T, k)
    dx = dXp[rows].sum(axis=1)
    if n_shared:
        dx = dx + dXp[T * k:T * k + T]
    dx = bf16_round(dx)
    pref = chunk_prefix(offsets)
    qd, sd = quant_128x1_grouped(dD, offsets)
    qh, sh = quant_128x1_grouped(h, offsets)
    dW_dn = grouped_wgrad(qd, sd, qh, sh, pref).astype(np.float32).astype(np.float64)
    qg, sg = quant_128x1_grouped(dGU, offsets)
    qx, sx = quant_128x1_grouped(x[np.asarray(perm_src, dtype=np.int64)], offsets)
    dW_gu = grouped_wgrad(qg, sg, qx, sx, pref).astype(np.float32).astype(np.float64)
    return dict(dx=dx, dw=cb["dw"], dW_gu=dW_gu, dW_dn=dW_dn, dD=dD, dh=dh, GU=GU, dGU=dGU,
                h=h, dXp=dXp)


# ---- router -----------------------------------------------------------------
#
# The gate weights are w_j = s_(e_j) / sum_i s_(e_i) over a token's selected
# experts, s = sigmoid(x . C_e) (the unbiased scores; the bias and the choice of
# experts carry no gradient - the bias only selects, section 无额外损耗的负载均衡
# of the news.qq.com article; the gating stays in FP32, section FP8 低精度训练).
# With S = sum_i s_(e_i):
#   ds_(e_i)     = (dw_i - sum_j dw_j w_j) / S
#   dlogit_(e_i) = ds_(e_i) s_(e_i) (1 - s_(e_i))
#   dx[t]        = sum_i dlogit_i C[e_i]           (the router's part of dx)
#   dC[e]        = sum over the (t, i) that chose e of dlogit_i x[t]


def router_backward(x_bits, centroids, idx, dw):
    """x bf16 bits [T, H]; centroids fp32 [E, H]; idx [T, k]; dw [T, k].
    float64 throughout (logits recomputed exactly).  Returns dict(dlogit [T, k],
    dx [T, H], dC [E, H])."""
    x = bf16_value_from_bits(x_bits)
    C = np.asarray(centroids, dtype=np.float32).astype(np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    dw = np.asarray(dw, dtype=np.float64)
    T, k = idx.shape
    logit = np.einsum("th,tkh->tk", x, C[idx])
    s = 1.0 / (1.0 + np.exp(-logit))
    S = s.sum(axis=1, keepdims=True)
    w = s / S
    ds = (dw - np.sum(dw * w, axis=1, keepdims=True)) / S
    dlogit = ds * s * (1.0 - s)
    dx = np.einsum("tk,tkh->th", dlogit, C[idx])
    dC = np.zeros_like(C)
    np.add.at(dC, idx.reshape(-1), dlogit.reshape(-1, 1) * np.repeat(x, k, axis=0))
    return dict(dlogit=dlogit, dx=dx, dC=dC)


def layer_backward(dy_bits, fwd: dict, wts, x_bits, centroids, T: int, k: int, I: int,
                   n_shared: int = 1, seq_len: int | None = None, alpha: float = 0.0001):
    """Whole-layer backward: expert_backward's results plus dlogit and dC from
    router_backward on its dw (router_backward_with_balance when the loss
    holds the sequence-wise balance term over runs of seq_len tokens), and
    dx_total = bf16(dx_expert + dx_router)."""
    eb = expert_backward(dy_bits, fwd, wts, x_bits, T, k, I, n_shared)
    if seq_len is None:
        rb = router_backward(x_bits, centroids, fwd["route"]["idx"], eb["dw"])
    else:
        rb = router_backward_with_balance(x_bits, centroids, fwd["route"]["idx"], eb["dw"],
                                          seq_len, alpha)
    out = dict(eb)
    out.update(dx_expert=eb["dx"], dx=bf16_round(eb["dx"] + rb["dx"]), dlogit=rb["dlogit"],
               dC=rb["dC"])
    return out


def router_backward_with_balance(x_bits, centroids, idx, dw, seq_len: int, alpha: float,
                                 dx_in=None):
    """The router's backward when the loss also holds the sequence-wise balance
    term alpha * sum_b L_bal,b (oracle.balance.seq_balance; f held fixed with
    the selection): the logits' gradient is the gate part of router_backward
    on the chosen experts plus seq_balance_grad_logits on every expert, and
    dx = dx_in + dlogit C, dC = dlogit^T x.  float64.  Returns dict(dlogit
    [T, E], dx [T, H], dC [E, H])."""
    from .balance import seq_balance_grad_logits
    from .route import router_scores
    x = bf16_value_from_bits(x_bits)
    C = np.asarray(centroids, dtype=np.float32).astype(np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    s, _ = router_scores(x_bits, centroids, np.zeros(C.shape[0], np.float32))
    g = seq_balance_grad_logits(s, idx, seq_len, alpha)
    gate = router_backward(x_bits, centroids, idx, dw)["dlogit"]
    rows = np.repeat(np.arange(T), k)
    np.add.at(g, (rows, idx.reshape(-1)), gate.reshape(-1))
    dx = g @ C
    if dx_in is not None:
        dx = dx + np.asarray(dx_in, dtype=np.float64)
    return dict(dlogit=g, dx=dx, dC=g.T @ x)
