"""Sequence-wise balance statistic on the GPU, through the C ABI.

* moe_route_scores: the routing outputs bit-identical to moe_route's on the
  same inputs; every expert's score within 4e-6 of the oracle's float64
  sigmoid (the bound the router's weights are held to: fp32-accumulated
  logits within a few 1e-6); score_sums within the fp32 sum bound of the
  GPU's own scores;
* moe_seq_balance on given scores: f bit-exact (fp32 of the exact rational
  E*count/(k*L)), P within its fp32 evaluation bound, the loss within the
  bound that P and the last reduction imply; ragged last sequence, a single
  sequence, seq_len 1, unchosen experts;
* MoELayer.forward(seq_len=...) on the mid config, and the same two calls at
  V3 shapes (T=16384, sequences of 4096), against the oracle's statistic on
  the GPU's own choice;
* moe_router_backward_dense (the router's backward with the balance term):
  dlogit against the oracle within 2^-14 of the token's gradient scale; dx
  and dC against the exact sums of the GPU's own dlogit within their fp32
  accumulation bounds (dx plus one bf16 rounding); ragged tiles, one and
  several token slices, with and without an incoming dx; and the layer's
  backward with seq_len end to end against the oracle's chain.
"""
import numpy as np
import pytest
import torch

import synth
import fp8_block_scaled_bias_amd as M
from gpu_common import bf16_dev, compare_routes, dev, host, log
from test_gpu_layer import build_layer
from oracle import backward as OBK
from oracle import balance as OB
from oracle import formats as OF
from oracle import layer as OL
from oracle import route as OR
from gpu_common import assert_within_one_bf16_ulp, bf16_values_host, rel_l2

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _f32(shape):
    return torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")


def _i32(shape):
    return torch.full(shape, -7, dtype=torch.int32, device="cuda")


def _seq_gpu(scores, ssum, idx, seq_len, alpha):
    T, E = scores.shape
    k = idx.shape[1]
    B = -(-T // seq_len)
    f, p, loss = _f32((B, E)), _f32((B, E)), _f32((B,))
    wsb = max(16, M.moe_seq_balance_workspace_bytes(T, E, seq_len))
    ws = torch.empty((wsb,), dtype=torch.uint8, device="cuda")
    M.moe_seq_balance(dev(np.ascontiguousarray(scores, np.float32)), dev(ssum), dev(idx), T, E, k,
                      seq_len, alpha, f, p, loss, ws, wsb)
    return host(f), host(p), host(loss)


def check_statistic(f, p, loss, scores, ssum, idx, seq_len, alpha, label):
    """GPU f, P, loss against the oracle on the scores the GPU read (float64
    sum per token) and the sums it divided by (within one fp32 rounding of
    theirs)."""
    T, E = scores.shape
    s64 = np.asarray(scores, np.float64)
    ref = OB.seq_balance(s64, idx, seq_len, alpha)
    assert np.array_equal(f, ref["f"].astype(np.float32)), label
    # P: each term s/S rounded once (plus S itself one rounding away from the
    # exact sum), then <= 64 + chunks additions and the division by L
    nch = -(-min(seq_len, T) // 64)
    relP = (64 + nch + 4) * U
    S_rel = np.abs(np.asarray(ssum, np.float64) - s64.sum(1)) / s64.sum(1)
    assert S_rel.max() <= (E + 2) * U, (label, S_rel.max())
    tolP = (relP + (E + 2) * U) * ref["P"] + 1e-30
    errP = np.abs(p - ref["P"])
    log(f"[seq balance] {label}: max |P err| / bound {float((errP / tolP).max()):.2e}")
    assert (errP <= tolP).all(), label
    # loss: sum_e f P with P as above, then E products and E additions
    tolL = alpha * np.sum(ref["f"] * tolP, 1) + (E + 4) * U * ref["loss"]
    errL = np.abs(loss - ref["loss"])
    log(f"[seq balance] {label}: loss {loss[:4]} max |err| / bound {float((errL / tolL).max()):.2e}")
    assert (errL <= tolL).all(), label


@pytest.mark.parametrize("T,E,k,seq_len", [(300, 16, 4, 128), (64, 256, 8, 64), (5, 8, 3, 1),
                                           (1000, 64, 6, 4096), (4100, 256, 8, 1024)])
def test_seq_balance_kernel(T, E, k, seq_len):
    rng = np.random.default_rng([T, E, k])
    scores = (1.0 / (1.0 + np.exp(-rng.standard_normal((T, E)) * 2))).astype(np.float32)
    idx = np.sort(np.stack([rng.choice(E // 2, k, replace=False) for _ in range(T)]), 1)
    idx = idx.astype(np.int32)      # the upper half of the experts is never chosen
    ssum = scores.astype(np.float64).sum(1).astype(np.float32)
    log(f"[seq balance] T={T} E={E} k={k} seq_len={seq_len}")
    f, p, loss = _seq_gpu(scores, ssum, idx, seq_len, 1e-4)
    check_statistic(f, p, loss, scores, ssum, idx, seq_len, 1e-4, f"T={T} L={seq_len}")
    assert not f[:, E // 2:].any()


def test_seq_balance_uniform_scores_give_alpha():
    T, E, k = 256, 32, 4
    rng = np.random.default_rng(2)
    scores = np.full((T, E), 0.5, np.float32)
    idx = np.sort(np.stack([rng.choice(E, k, replace=False) for _ in range(T)]), 1).astype(np.int32)
    f, p, loss = _seq_gpu(scores, np.full(T, 16.0, np.float32), idx, 100, 1e-4)
    np.testing.assert_allclose(loss, 1e-4, rtol=8 * E * U)
    assert np.all(p == np.float32(1.0 / E))


@pytest.mark.parametrize("name,T", [("tiny", 64), ("mid", 200), ("decode", 128)])
def test_route_scores(name, T):
    cfg = synth.CONFIGS[name]
    bits = synth.gen_x(cfg, seed=3, T=T)
    C = synth.gen_centroids(cfg, seed=3)
    b = synth.gen_bias(cfg, seed=3)
    E, k = cfg.E, cfg.k
    wsb = max(16, M.moe_route_workspace_bytes(T, cfg.H, E))
    ws = torch.empty((wsb,), dtype=torch.uint8, device="cuda")
    outs = []
    for with_scores in (False, True):
        idx, w, cnt = _i32((T, k)), _f32((T, k)), _i32((E,))
        sc, ss = _f32((T, E)), _f32((T,))
        args = (bf16_dev(bits), T, cfg.H, dev(C), dev(b), E, cfg.n_group, cfg.topk_group, k, idx,
                w, cnt, ws, wsb)
        if with_scores:
            M.moe_route_scores(*args, sc, ss)
        else:
            M.moe_route(*args)
        outs.append((host(idx), host(w), host(cnt), host(sc), host(ss)))
    for a, b_ in zip(outs[0][:3], outs[1][:3]):
        assert np.array_equal(a.view(np.uint32), b_.view(np.uint32))
    sc, ss = outs[1][3], outs[1][4]
    s_ref, _ = OR.router_scores(bits, C, b)
    err = np.abs(sc - s_ref)
    log(f"[route scores] {name}: max |s_gpu - s_oracle| = {err.max():.3e}")
    assert err.max() <= 4e-6
    own = sc.astype(np.float64).sum(1)
    assert (np.abs(ss - own) <= (E + 2) * U * own).all()


def test_layer_seq_balance_mid():
    cfg = synth.MID
    layer, C, b = build_layer(cfg)
    x = synth.gen_x(cfg)
    log(f"[layer seq balance] mid: T={cfg.T}, seq_len 64")
    layer.forward(bf16_dev(x), seq_len=64)
    bufs = layer.buffers(cfg.T)
    torch.cuda.synchronize()
    ora = OR.route(x, C, b, cfg.n_group, cfg.topk_group, cfg.k)
    assert len(compare_routes(host(bufs.topk_idx), ora, "mid")) == 0
    s_ref, _ = OR.router_scores(x, C, b)
    _check_layer(bufs, s_ref, host(bufs.topk_idx), 64, cfg, "mid")


def _check_layer(bufs, s_ref, idx, seq_len, cfg, label):
    """The layer's statistic against the oracle on the GPU's own choice, with
    the score error (<= 4e-6 per score) carried into P and the loss."""
    ref = OB.seq_balance(s_ref, idx, seq_len, 1e-4)
    f, p, loss = host(bufs.seq_f), host(bufs.seq_p), host(bufs.seq_loss)
    assert np.array_equal(f, ref["f"].astype(np.float32)), label
    # s' = s/S moves by at most (4e-6 + s' * E * 4e-6) / S per token
    S = s_ref.sum(1, keepdims=True)
    ds = (4e-6 + (s_ref / S) * cfg.E * 4e-6) / S
    B = len(loss)
    tolP = np.stack([ds[i * seq_len:(i + 1) * seq_len].mean(0) for i in range(B)])
    tolP = tolP + 1e-5 * ref["P"]
    errP = np.abs(p - ref["P"])
    log(f"[layer seq balance] {label}: loss {loss[:4]}, max |P err| / bound "
        f"{float((errP / tolP).max()):.2e}")
    assert (errP <= tolP).all(), label
    tolL = 1e-4 * np.sum(ref["f"] * tolP, 1) + 1e-5 * ref["loss"]
    assert (np.abs(loss - ref["loss"]) <= tolL).all(), label


def test_seq_balance_v3_prefill():
    """V3 shapes, T=16384 in sequences of 4096, the calls the layer makes."""
    cfg = synth.PREFILL
    T, E, k = cfg.T, cfg.E, cfg.k
    x = synth.gen_x(cfg)
    C, b = synth.gen_centroids(cfg), synth.gen_bias(cfg)
    log(f"[seq balance] V3 prefill: T={T}, seq_len 4096")
    wsb = max(16, M.moe_route_workspace_bytes(T, cfg.H, E))
    ws = torch.empty((wsb,), dtype=torch.uint8, device="cuda")
    idx, w, cnt, sc, ss = _i32((T, k)), _f32((T, k)), _i32((E,)), _f32((T, E)), _f32((T,))
    M.moe_route_scores(bf16_dev(x), T, cfg.H, dev(C), dev(b), E, cfg.n_group, cfg.topk_group, k,
                       idx, w, cnt, ws, wsb, sc, ss)

    class Bufs:
        pass
    bufs = Bufs()
    B = T // 4096
    bufs.seq_f, bufs.seq_p, bufs.seq_loss = _f32((B, E)), _f32((B, E)), _f32((B,))
    swb = M.moe_seq_balance_workspace_bytes(T, E, 4096)
    sw = torch.empty((swb,), dtype=torch.uint8, device="cuda")
    M.moe_seq_balance(sc, ss, idx, T, E, k, 4096, 1e-4, bufs.seq_f, bufs.seq_p, bufs.seq_loss, sw,
                      swb)
    torch.cuda.synchronize()
    s_ref, _ = OR.router_scores(x, C, b)
    assert np.abs(host(sc) - s_ref).max() <= 4e-6
    _check_layer(bufs, s_ref, host(idx), 4096, cfg, "V3 prefill")


def check_dense_router(xbits, C, idx, dw, scores, ssum, seq_len, alpha, dx_in, dl, dx, dC, label,
                       extra_rel=0.0):
    """GPU dlogit [T, E], dx (bf16 values) and dC against the oracle (dlogit)
    and the exact sums of the GPU's own dlogit (dx, dC).  extra_rel widens
    the dlogit bound when the scores themselves carry the router's error."""
    T, k = idx.shape
    E = C.shape[0]
    ref = OBK.router_backward_with_balance(xbits, C, idx, dw, seq_len, alpha)
    s64 = np.asarray(scores, np.float64)
    sel = np.take_along_axis(s64, idx.astype(np.int64), 1)
    Ssel = sel.sum(1)
    dw64 = np.abs(np.asarray(dw, np.float64))
    st = OB.seq_balance(s64, idx, seq_len, alpha)
    Lb = np.array([min(seq_len, T - (t // seq_len) * seq_len) for t in range(T)], np.float64)
    fmax = st["f"].max(1)[np.arange(T) // seq_len]
    scale = (dw64.max(1) + np.sum(dw64 * sel, 1) / Ssel) / Ssel + abs(alpha) / Lb * fmax / s64.sum(1)
    err = np.abs(dl - ref["dlogit"])
    tol = (2.0 ** -14 + extra_rel) * scale[:, None]
    log(f"[dense router] {label}: max |dlogit err| / bound {float((err / tol).max()):.2e}")
    assert (err <= tol).all(), label
    Cd = np.asarray(C, np.float32).astype(np.float64)
    dl64 = np.asarray(dl, np.float64)
    base = np.zeros((T, Cd.shape[1])) if dx_in is None else np.asarray(dx_in, np.float64)
    exact = base + dl64 @ Cd
    acc = (E + 2) * 2.0 ** -24 * (np.abs(base) + np.abs(dl64) @ np.abs(Cd))
    assert_within_one_bf16_ulp(dx, exact, f"{label} dx", acc)
    xv = OF.bf16_value_from_bits(xbits)
    exC = dl64.T @ xv
    bndC = (1024 + 16 + 2) * 2.0 ** -24 * (np.abs(dl64).T @ np.abs(xv)) + 1e-30
    ratio = np.abs(np.asarray(dC, np.float64) - exC) / bndC
    log(f"[dense router] {label}: max |dC err| / bound {float(ratio.max()):.2e}")
    assert (ratio <= 1).all(), label


@pytest.mark.parametrize("T,H,E,k,seq_len,mode", [(300, 256, 16, 4, 128, "dx_in"),
                                                  (2100, 1024, 64, 8, 1000, "none"),
                                                  (130, 7168, 256, 8, 4096, "dx_in")])
def test_router_backward_dense_kernel(T, H, E, k, seq_len, mode):
    rng = np.random.default_rng([T, H, E])
    xbits = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    C = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    idx = np.sort(np.stack([rng.choice(E, k, replace=False) for _ in range(T)]), 1).astype(np.int32)
    dw = rng.standard_normal((T, k)).astype(np.float32)
    s_ref, _ = OR.router_scores(xbits, C, np.zeros(E, np.float32))
    scores = s_ref.astype(np.float32)
    ssum = scores.astype(np.float64).sum(1).astype(np.float32)
    alpha = 0.05
    f = OB.seq_balance(scores.astype(np.float64), idx, seq_len, alpha)["f"].astype(np.float32)
    dx_in = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32)) if mode == "dx_in" else None
    log(f"[dense router] T={T} H={H} E={E} k={k} seq_len={seq_len} {mode}")
    wsb = max(16, M.moe_router_backward_dense_workspace_bytes(T, H, E))
    ws = torch.empty((wsb,), dtype=torch.uint8, device="cuda")
    dx = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    dC, dl = _f32((E, H)), _f32((T, E))
    M.moe_router_backward_dense(bf16_dev(xbits), dev(C), dev(idx), dev(dw), dev(scores), dev(ssum),
                                dev(f), T, H, E, k, seq_len, alpha,
                                None if dx_in is None else bf16_dev(dx_in), dx, dC, dl, ws, wsb)
    torch.cuda.synchronize()
    check_dense_router(xbits, C, idx, dw, scores, ssum, seq_len, alpha,
                       None if dx_in is None else OF.bf16_value_from_bits(dx_in), host(dl),
                       bf16_values_host(dx), host(dC), f"T={T} E={E}")


def test_layer_backward_with_balance_mid():
    """MoELayer.forward and backward with seq_len on the mid config: the
    router stage against the oracle on the GPU's own dw, scores and dx, then
    dx_total and dC end to end against the oracle's chain."""
    cfg = synth.MID
    T, k, I, L_ = cfg.T, cfg.k, cfg.I, 64
    alpha = 0.5
    layer, C, b = build_layer(cfg)
    x = synth.gen_x(cfg)
    dy = synth.gen_dy(cfg)
    log(f"[layer bwd balance] mid: T={T}, seq_len {L_}, alpha {alpha}")
    x_d = bf16_dev(x)
    layer.forward(x_d, seq_len=L_, alpha=alpha)
    bufs = layer.buffers(T)
    bb = layer.backward(bf16_dev(dy), x_d, seq_len=L_, alpha=alpha)
    torch.cuda.synchronize()
    idx = host(bufs.topk_idx)
    fwd = OL.layer(x, C, b, _oracle_weights(cfg), cfg.n_group, cfg.topk_group, k, I)
    assert len(compare_routes(idx, fwd["route"], "mid")) == 0
    # the scores carry the router's error (<= 4e-6 each): widen the bound
    check_dense_router(x, C, idx, host(bb.dw), host(bufs.scores), host(bufs.score_sums), L_, alpha,
                       bf16_values_host(bb.dx), host(bb.dlogit), bf16_values_host(bb.dx_total),
                       host(bb.dC), "mid layer", extra_rel=1e-4)
    ref = OBK.layer_backward(dy, fwd, _oracle_weights(cfg), x, C, T, k, I, seq_len=L_, alpha=alpha)
    errs = dict(dx=rel_l2(bf16_values_host(bb.dx_total), ref["dx"]),
                dC=rel_l2(host(bb.dC), ref["dC"]))
    log(f"[layer bwd balance] mid: end to end " + ", ".join(f"{k_} {v:.2e}" for k_, v in errs.items()))
    assert max(errs.values()) <= 5e-3, errs


def _oracle_weights(cfg):
    from test_gpu_layer import oracle_weights
    return oracle_weights(cfg)


def test_router_backward_dense_v3_prefill_sampled():
    """V3 shapes at T=16384 in sequences of 4096 (the benchmark's batch): the
    GPU's routing, scores and statistic, dw N(0,1), alpha = 1e-4; dlogit and
    dx on 48 sampled tokens, dC on 4 sampled experts (over every token)."""
    cfg = synth.PREFILL
    T, H, E, k, L_ = cfg.T, cfg.H, cfg.E, cfg.k, 4096
    alpha = 1e-4
    x = synth.gen_x(cfg)
    C, b = synth.gen_centroids(cfg), synth.gen_bias(cfg)
    log(f"[dense router] V3 prefill T={T}: route with scores, statistic, backward")
    wsb = max(16, M.moe_route_workspace_bytes(T, H, E))
    ws = torch.empty((wsb,), dtype=torch.uint8, device="cuda")
    idx, w, cnt, sc, ss = _i32((T, k)), _f32((T, k)), _i32((E,)), _f32((T, E)), _f32((T,))
    x_d, C_d = bf16_dev(x), dev(C)
    M.moe_route_scores(x_d, T, H, C_d, dev(b), E, cfg.n_group, cfg.topk_group, k, idx, w, cnt, ws,
                       wsb, sc, ss)
    B = T // L_
    f, p, loss = _f32((B, E)), _f32((B, E)), _f32((B,))
    swb = M.moe_seq_balance_workspace_bytes(T, E, L_)
    sw = torch.empty((swb,), dtype=torch.uint8, device="cuda")
    M.moe_seq_balance(sc, ss, idx, T, E, k, L_, alpha, f, p, loss, sw, swb)
    dw = np.random.default_rng(12).standard_normal((T, k)).astype(np.float32)
    dx_in = synth.gen_dy(cfg)
    dwb = max(16, M.moe_router_backward_dense_workspace_bytes(T, H, E))
    dws = torch.empty((dwb,), dtype=torch.uint8, device="cuda")
    dx = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    dC, dl = _f32((E, H)), _f32((T, E))
    M.moe_router_backward_dense(x_d, C_d, idx, dev(dw), sc, ss, f, T, H, E, k, L_, alpha,
                                bf16_dev(dx_in), dx, dC, dl, dws, dwb)
    torch.cuda.synchronize()
    rng = np.random.default_rng(13)
    toks = np.sort(np.concatenate([[0, L_ - 1, L_, T - 1], rng.choice(T, 44, replace=False)]))
    idx_h, dl_h, sc_h, f_h = host(idx), host(dl), host(sc), host(f)
    s_ref, _ = OR.router_scores(x[toks], C, b)
    # dlogit on the sampled tokens: the oracle's formulas on exact scores with
    # the GPU's f (the statistic is checked on its own elsewhere)
    sel = np.take_along_axis(s_ref, idx_h[toks].astype(np.int64), 1)
    Ssel = sel.sum(1, keepdims=True)
    dwt = dw[toks].astype(np.float64)
    gate = (dwt - np.sum(dwt * sel / Ssel, 1, keepdims=True)) / Ssel * sel * (1 - sel)
    S = s_ref.sum(1, keepdims=True)
    fb = f_h[toks // L_].astype(np.float64)
    ref = alpha / L_ * (fb - np.sum(fb * s_ref / S, 1, keepdims=True)) / S * s_ref * (1 - s_ref)
    np.add.at(ref, (np.repeat(np.arange(len(toks)), k), idx_h[toks].reshape(-1)), gate.reshape(-1))
    scale = (np.abs(dwt).max(1) + np.sum(np.abs(dwt) * sel, 1) / Ssel[:, 0]) / Ssel[:, 0] \
        + alpha / L_ * fb.max(1) / S[:, 0]
    err = np.abs(dl_h[toks] - ref)
    log(f"[dense router] V3: max |dlogit err| / scale {float((err / scale[:, None]).max()):.2e}")
    assert (err <= (2.0 ** -14 + 1e-4) * scale[:, None]).all()
    # dx on the sampled tokens from the GPU's own dlogit
    Cd = C.astype(np.float64)
    dl64 = dl_h[toks].astype(np.float64)
    base = OF.bf16_value_from_bits(dx_in[toks])
    exact = base + dl64 @ Cd
    acc = (E + 2) * 2.0 ** -24 * (np.abs(base) + np.abs(dl64) @ np.abs(Cd))
    assert_within_one_bf16_ulp(bf16_values_host(dx)[toks], exact, "V3 dense dx", acc)
    # dC on sampled experts over every token
    xv = OF.bf16_value_from_bits(x)
    dCh = host(dC).astype(np.float64)
    for e in [0, 255] + list(rng.choice(E, 2, replace=False)):
        col = dl_h[:, e].astype(np.float64)
        ex = col @ xv
        bnd = (1024 + 16 + 2) * 2.0 ** -24 * (np.abs(col) @ np.abs(xv)) + 1e-30
        assert (np.abs(dCh[e] - ex) <= bnd).all(), e
