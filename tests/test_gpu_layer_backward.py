"""Backward of the layer's expert path on the GPU, through the C ABI.

* moe_combine_backward: dD bit-exact (bf16 of the fp32 product w * dy on both
  sides; the shared rows are dy itself), dw within the fp32 accumulation
  bound H * 2^-23 * sum |dy D|;
* swiglu_backward: dg, du and h within one bf16 ulp of the FP64 values (the
  GPU evaluates in fp32, then rounds once to bf16);
* moe_router_backward / moe_router_dcentroids: dlogit against the oracle's
  float64 router backward within 2^-14 of the token's gradient scale (the
  GPU recomputes the logits in fp32); dx and dC against the exact sums of
  the GPU's own dlogit, within one bf16 ulp plus the fp32 accumulation bound
  (dx) and within the fp32 accumulation bound (dC);
* MoELayer.backward on the tiny and mid configs: every stage against the
  oracle applied to the GPU's own inputs to that stage (dD, every E4M3 code
  and scale, both operand layouts bit-exact; GEMM outputs within the grouped
  GEMM's derived bound plus one bf16 rounding; SwiGLU backward within one
  bf16 ulp; weight gradients within the wgrad bound; the router stage as
  above), then dx, dw, dC, dW_gu and dW_dn against the oracle's independent
  chain (oracle.backward.layer_backward after oracle.layer) within relative
  L2 5e-3.
"""
import numpy as np
import pytest
import torch

import synth
import fp8_block_scaled_bias_amd as M
from gpu_common import (assert_within_one_bf16_ulp, bf16_dev, bf16_ulp, bf16_values_host,
                        compare_routes, dev, host, log, rel_l2)
from test_gpu_kernels import gemm_accumulation_bound
from test_gpu_layer import build_layer, oracle_weights
from oracle import backward as OBK
from oracle import combine as OC
from oracle import formats as OF
from oracle import gemm as OG
from oracle import layer as OL
from oracle import quant as OQ

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,k,H,ns", [(37, 8, 1024, 1), (5, 3, 256, 0), (64, 4, 7168, 1)])
def test_combine_backward_kernel(T, k, H, ns):
    rng = np.random.default_rng([T, k, H])
    R = T * k + ns * T
    dy = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    D = synth.f32_to_bf16_bits(rng.standard_normal((R, H)).astype(np.float32))
    inv_perm = rng.permutation(T * k).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    log(f"[combine bwd] T={T} k={k} H={H} shared={ns}")
    dD = torch.full((R, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    dw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    M.moe_combine_backward(bf16_dev(dy), dev(inv_perm), dev(w), bf16_dev(D), T, k, H, ns, dD, dw)
    dyv, Dv = OF.bf16_value_from_bits(dy), OF.bf16_value_from_bits(D)
    ref = OBK.combine_backward(dyv, Dv, inv_perm, w, T, k, ns)
    assert np.array_equal(bf16_values_host(dD), ref["dD"])
    rows = inv_perm.reshape(T, k).astype(np.int64)
    bound = H * 2.0 ** -23 * np.stack([np.sum(np.abs(dyv * Dv[rows[:, j]]), axis=1) for j in range(k)], 1)
    assert (np.abs(host(dw) - ref["dw"]) <= bound).all()


@pytest.mark.parametrize("M_,I", [(300, 128), (7, 2048)])
def test_swiglu_backward_kernel(M_, I):
    rng = np.random.default_rng([M_, I])
    gu = rng.standard_normal((M_, 2 * I)).astype(np.float32) * 3.0
    gu[0, :8] = [0.0, -0.0, 20.0, -20.0, 80.0, -80.0, 1e-3, -1e-3]
    gub = synth.f32_to_bf16_bits(gu)
    dh = synth.f32_to_bf16_bits(rng.standard_normal((M_, I)).astype(np.float32))
    log(f"[swiglu bwd] M={M_} I={I}")
    dgu = torch.empty((M_, 2 * I), dtype=torch.bfloat16, device="cuda")
    h = torch.empty((M_, I), dtype=torch.bfloat16, device="cuda")
    M.swiglu_backward(bf16_dev(gub), bf16_dev(dh), M_, I, dgu, h)
    r_dgu, r_h = OBK.swiglu_backward(OF.bf16_value_from_bits(gub), OF.bf16_value_from_bits(dh), I)
    for got, ref, what in ((bf16_values_host(dgu), r_dgu, "dgu"), (bf16_values_host(h), r_h, "h")):
        d = np.abs(got - ref)
        assert (d <= bf16_ulp(np.maximum(np.abs(got), np.abs(ref))) + 1e-30).all(), what


@pytest.mark.parametrize("T,k,H,ns", [(37, 8, 1024, 1), (5, 3, 256, 0), (64, 4, 7168, 1)])
def test_combine_backward_writes_1x128_codes(T, k, H, ns):
    """The 1x128 codes and scales moe_combine_backward writes with dD equal
    the oracle's quant_1x128 of dD as stored, and fp8_quant_1x128 of the same
    bf16 rows, bit for bit (rows of both kinds: routed w*dy and shared dy)."""
    rng = np.random.default_rng([T, k, H, 1])
    R = T * k + ns * T
    dy = rng.standard_normal((T, H)).astype(np.float32)
    dy[0, :128] = 0.0                                   # an all-zero tile
    dy = synth.f32_to_bf16_bits(dy)
    D = synth.f32_to_bf16_bits(rng.standard_normal((R, H)).astype(np.float32))
    inv_perm = rng.permutation(T * k).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    dD = torch.empty((R, H), dtype=torch.bfloat16, device="cuda")
    dw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    q = torch.empty((R, H), dtype=torch.uint8, device="cuda")
    sc = torch.empty((R, H // 128), dtype=torch.float32, device="cuda")
    M.moe_combine_backward(bf16_dev(dy), dev(inv_perm), dev(w), bf16_dev(D), T, k, H, ns, dD, dw,
                           d_expert_out_e4m3=q, d_expert_out_scale=sc)
    oq, os_ = OQ.quant_1x128(bf16_values_host(dD).astype(np.float32))
    assert np.array_equal(host(q), oq) and np.array_equal(host(sc), os_)
    q2 = torch.empty_like(q)
    s2 = torch.empty_like(sc)
    M.fp8_quant_1x128(dD, R, H, H, 0, q2, s2)
    assert torch.equal(q, q2) and torch.equal(sc, s2)


@pytest.mark.parametrize("M_,I", [(300, 128), (7, 2048)])
def test_swiglu_backward_writes_1x128_codes(M_, I):
    """The 1x128 codes and scales swiglu_backward writes with dGU equal the
    oracle's quant_1x128 of dGU as stored, and fp8_quant_1x128 of the same
    bf16 rows, bit for bit (dg and du halves)."""
    rng = np.random.default_rng([M_, I, 1])
    gub = synth.f32_to_bf16_bits(rng.standard_normal((M_, 2 * I)).astype(np.float32) * 3.0)
    dh = rng.standard_normal((M_, I)).astype(np.float32)
    dh[1, :] = 0.0                                      # zero tiles in both halves
    dh = synth.f32_to_bf16_bits(dh)
    dgu = torch.empty((M_, 2 * I), dtype=torch.bfloat16, device="cuda")
    h = torch.empty((M_, I), dtype=torch.bfloat16, device="cuda")
    q = torch.empty((M_, 2 * I), dtype=torch.uint8, device="cuda")
    sc = torch.empty((M_, 2 * I // 128), dtype=torch.float32, device="cuda")
    M.swiglu_backward(bf16_dev(gub), bf16_dev(dh), M_, I, dgu, h, dgu_e4m3=q, dgu_scale=sc)
    oq, os_ = OQ.quant_1x128(bf16_values_host(dgu).astype(np.float32))
    assert np.array_equal(host(q), oq) and np.array_equal(host(sc), os_)
    q2 = torch.empty_like(q)
    s2 = torch.empty_like(sc)
    M.fp8_quant_1x128(dgu, M_, 2 * I, 2 * I, 0, q2, s2)
    assert torch.equal(q, q2) and torch.equal(sc, s2)


@pytest.mark.parametrize("sizes,I", [([300, 0, 1, 129, 128, 77], 256), ([40, 2, 250], 2048)],
                         ids=["ragged", "wide_I"])
def test_swiglu_backward_grouped_equals_unfused(sizes, I):
    """swiglu_backward_grouped writes what swiglu_backward, fp8_quant_1x128 and
    fp8_quant_128x1_grouped write on the same rows, bit for bit (groups that are
    empty, one row, exactly one chunk, ragged), and its 128x1 codes of dGU and
    h equal the oracle's grouped quantiser of the stored bf16 values."""
    from test_gpu_wgrad import _to_logical
    G = len(sizes)
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    Mt = int(offs[-1])
    rng = np.random.default_rng([Mt, I])
    gu = rng.standard_normal((Mt, 2 * I)).astype(np.float32) * 3.0
    dh = rng.standard_normal((Mt, I)).astype(np.float32)
    dh[5, :] = 0.0                                      # zero tiles, both layouts
    gub, dhb = bf16_dev(synth.f32_to_bf16_bits(gu)), bf16_dev(synth.f32_to_bf16_bits(dh))
    offs_d = dev(offs.astype(np.int32))
    cap = M.wgrad_chunks(Mt, G)
    u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16
    dgu = torch.empty((Mt, 2 * I), dtype=bf, device="cuda")
    h = torch.empty((Mt, I), dtype=bf, device="cuda")
    q = torch.empty((Mt, 2 * I), dtype=u8, device="cuda")
    qs = torch.empty((Mt, 2 * I // 128), dtype=f32, device="cuda")
    cg, sg = (torch.zeros((cap, 2 * I, 128), dtype=u8, device="cuda"),
              torch.zeros((cap, 2 * I), dtype=f32, device="cuda"))
    ch, sh = (torch.zeros((cap, I, 128), dtype=u8, device="cuda"),
              torch.zeros((cap, I), dtype=f32, device="cuda"))
    log(f"[swiglu bwd grouped] sizes {sizes} I={I}")
    M.swiglu_backward_grouped(gub, dhb, offs_d, G, Mt, I, dgu, h, q, qs, cap, cg, sg, ch, sh)
    # the unfused chain on the same inputs
    dgu2, h2 = torch.empty_like(dgu), torch.empty_like(h)
    M.swiglu_backward(gub, dhb, Mt, I, dgu2, h2)
    q2, qs2 = torch.empty_like(q), torch.empty_like(qs)
    M.fp8_quant_1x128(dgu2, Mt, 2 * I, 2 * I, 0, q2, qs2)
    cg2, sg2, ch2, sh2 = (torch.zeros_like(t) for t in (cg, sg, ch, sh))
    M.fp8_quant_128x1_grouped(dgu2, 2 * I, None, offs_d, G, Mt, 2 * I, cg2, sg2, cap)
    M.fp8_quant_128x1_grouped(h2, I, None, offs_d, G, Mt, I, ch2, sh2, cap)
    nch = int(OQ.chunk_prefix(offs)[-1])
    assert torch.equal(dgu.view(torch.int16), dgu2.view(torch.int16))
    assert torch.equal(h.view(torch.int16), h2.view(torch.int16))
    assert torch.equal(q, q2) and torch.equal(qs, qs2)
    assert torch.equal(cg[:nch], cg2[:nch]) and torch.equal(sg[:nch], sg2[:nch])
    assert torch.equal(ch[:nch], ch2[:nch]) and torch.equal(sh[:nch], sh2[:nch])
    for c, sc, ref in ((cg, sg, dgu), (ch, sh, h)):
        qo, so = OQ.quant_128x1_grouped(bf16_values_host(ref).astype(np.float32), offs)
        ql, sl = _to_logical(host(c), host(sc), qo.shape[1] // 128)
        assert np.array_equal(ql, qo) and np.array_equal(sl, so)
    # without the optional bf16 outputs: the same codes and scales
    q3, qs3 = torch.empty_like(q), torch.empty_like(qs)
    cg3, sg3, ch3, sh3 = (torch.zeros_like(t) for t in (cg, sg, ch, sh))
    M.swiglu_backward_grouped(gub, dhb, offs_d, G, Mt, I, None, None, q3, qs3, cap, cg3, sg3, ch3, sh3)
    assert torch.equal(q3, q) and torch.equal(qs3, qs)
    assert torch.equal(cg3, cg) and torch.equal(sg3, sg) and torch.equal(ch3, ch) and torch.equal(sh3, sh)


def _expert_rows(idx, E):
    """perm_src, inv_perm [T*k] and offsets [E+1] in moe_permute's layout: rows
    grouped by expert, each expert's tokens in ascending order."""
    T, k = idx.shape
    perm_src, inv_perm, offs = [], np.zeros(T * k, np.int32), [0]
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if idx[t, j] == e:
                    inv_perm[t * k + j] = len(perm_src)
                    perm_src.append(t)
        offs.append(len(perm_src))
    return np.array(perm_src, np.int32), inv_perm, np.array(offs, np.int32)


def check_router_stage(xbits, C, idx, dw32, inv_perm, perm_src, offs, dx_in, dl_rows, dx_out,
                       dC, label):
    """dl_rows (fp32 [T*k], expert-row order), dx_out (bf16 values), dC (fp32,
    or None to skip it) from the GPU; dx_in (bf16 values or None) and the
    rest its inputs."""
    T, k = idx.shape
    xv = OF.bf16_value_from_bits(xbits)
    C64 = np.asarray(C, np.float32).astype(np.float64)
    ref = OBK.router_backward(xbits, C, idx, dw32)
    dl = np.asarray(dl_rows, np.float64)[inv_perm.astype(np.int64)].reshape(T, k)
    # dlogit: the GPU's fp32 logits are within ~1e-6 relative of the exact
    # ones; dlogit moves by at most the token's gradient scale times that
    s = 1.0 / (1.0 + np.exp(-np.einsum("th,tkh->tk", xv, C64[idx])))
    S = s.sum(1, keepdims=True)
    dw64 = np.asarray(dw32, np.float64)
    scale = (np.abs(dw64).max(1, keepdims=True) + np.sum(np.abs(dw64) * s / S, 1, keepdims=True)) / S
    err = np.abs(dl - ref["dlogit"])
    log(f"[{label}] dlogit: max |err| / scale {float((err / scale).max()):.2e}")
    assert (err <= 2.0 ** -14 * scale).all(), label
    # dx from the GPU's own dlogit: exact sum, one bf16 rounding, fp32 fmas
    base = np.zeros((T, C64.shape[1])) if dx_in is None else np.asarray(dx_in, np.float64)
    terms = dl[:, :, None] * C64[idx]
    exact = base + terms.sum(1)
    acc = (k + 1) * 2.0 ** -23 * (np.abs(base) + np.abs(terms).sum(1))
    assert_within_one_bf16_ulp(dx_out, exact, f"{label} dx", acc)
    if dC is None:
        return
    # dC: each expert's rows in row order, fp32 fmas
    E = len(offs) - 1
    dC = np.asarray(dC, np.float64)
    dlr = np.asarray(dl_rows, np.float64)
    for e in range(E):
        r0, r1 = int(offs[e]), int(offs[e + 1])
        t_ = perm_src[r0:r1].astype(np.int64)
        prod = dlr[r0:r1, None] * xv[t_]
        ex = prod.sum(0)
        bnd = (r1 - r0 + 1) * 2.0 ** -24 * np.abs(prod).sum(0)
        assert (np.abs(dC[e] - ex) <= bnd).all(), f"{label} dC expert {e}"
    assert rel_l2(dC, ref["dC"]) <= 1e-4, (label, rel_l2(dC, ref["dC"]))


@pytest.mark.parametrize("T,H,E,k,mode,given", [(37, 1024, 64, 8, "dx_in", False),
                                                (5, 256, 16, 3, "none", False),
                                                (64, 7168, 256, 8, "in_place", False),
                                                (37, 1024, 64, 8, "dx_in", True),
                                                (64, 7168, 256, 8, "in_place", True)])
def test_router_backward_kernel(T, H, E, k, mode, given):
    """given: the chosen experts' scores come in as topk_s (the fp64 scores
    rounded to fp32, as the forward's fp32 scores are within an ulp of them)
    instead of being computed again from x and C."""
    rng = np.random.default_rng([T, H, E, k])
    xbits = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    C = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    idx = np.sort(np.stack([rng.choice(E, k, replace=False) for _ in range(T)]), 1).astype(np.int32)
    dw = rng.standard_normal((T, k)).astype(np.float32)
    perm_src, inv_perm, offs = _expert_rows(idx, E)
    log(f"[router bwd] T={T} H={H} E={E} k={k} {mode}; experts with no rows: "
        f"{int((np.diff(offs) == 0).sum())}")
    dx_in = None if mode == "none" else synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    x_d, C_d = bf16_dev(xbits), dev(C)
    dx_in_d = None if dx_in is None else bf16_dev(dx_in)
    dx_out = dx_in_d if mode == "in_place" else torch.full((T, H), float("nan"), dtype=torch.bfloat16,
                                                          device="cuda")
    dl_rows = torch.full((T * k,), float("nan"), dtype=torch.float32, device="cuda")
    dC = torch.full((E, H), float("nan"), dtype=torch.float32, device="cuda")
    ts = None
    if given:
        lg = np.einsum("th,tkh->tk", OF.bf16_value_from_bits(xbits),
                       C.astype(np.float64)[idx.astype(np.int64)])
        ts = dev((1.0 / (1.0 + np.exp(-lg))).astype(np.float32))
    M.moe_router_backward(x_d, C_d, dev(idx), dev(dw), dev(inv_perm), dx_in_d, T, H, E, k, dx_out,
                          dl_rows, topk_s=ts)
    M.moe_router_dcentroids(x_d, dev(perm_src), dev(offs), dl_rows, T, H, E, dC)
    torch.cuda.synchronize()
    check_router_stage(xbits, C, idx, dw, inv_perm, perm_src, offs,
                       None if dx_in is None else OF.bf16_value_from_bits(dx_in), host(dl_rows),
                       bf16_values_host(dx_out), host(dC), f"router bwd T={T}")
    assert not host(dC)[np.diff(offs) == 0].any()


def test_router_backward_v3_prefill_sampled():
    """V3 shapes at T=16384 (the benchmark's batch): the GPU's own routing and
    permutation, dw N(0,1); dlogit and dx on 64 sampled tokens, dC on 8
    sampled experts, each against the oracle / the exact sums of the GPU's
    dlogit as in check_router_stage."""
    from test_gpu_kernels import _permute_gpu
    cfg = synth.PREFILL
    T, H, E, k = cfg.T, cfg.H, cfg.E, cfg.k
    x = synth.gen_x(cfg)
    C, b = synth.gen_centroids(cfg), synth.gen_bias(cfg)
    log(f"[router bwd] V3 prefill T={T}: route, permute, backward")
    wsb = max(16, M.moe_route_workspace_bytes(T, H, E))
    ws = torch.empty((wsb,), dtype=torch.uint8, device="cuda")
    idx_d = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w_d = torch.empty((T, k), dtype=torch.float32, device="cuda")
    cnt_d = torch.empty((E,), dtype=torch.int32, device="cuda")
    x_d, C_d = bf16_dev(x), dev(C)
    ts_d = torch.empty((T, k), dtype=torch.float32, device="cuda")
    M.moe_route(x_d, T, H, C_d, dev(b), E, cfg.n_group, cfg.topk_group, k, idx_d, w_d, cnt_d, ws, wsb,
                topk_s=ts_d)
    idx = host(idx_d)
    offs, perm_src, inv_perm = _permute_gpu(idx, E, 0)
    dw = np.random.default_rng(8).standard_normal((T, k)).astype(np.float32)
    dx_in = synth.gen_dy(cfg)
    dx_out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    dl_rows = torch.empty((T * k,), dtype=torch.float32, device="cuda")
    dC = torch.empty((E, H), dtype=torch.float32, device="cuda")
    M.moe_router_backward(x_d, C_d, idx_d, dev(dw), dev(inv_perm), bf16_dev(dx_in), T, H, E, k,
                          dx_out, dl_rows, topk_s=ts_d)   # the forward's scores, as the layer
    M.moe_router_dcentroids(x_d, dev(perm_src), dev(offs), dl_rows, T, H, E, dC)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    toks = np.concatenate([[0, T - 1], rng.choice(T, 62, replace=False)])
    dlr = host(dl_rows)
    xs = x[toks]
    # dlogit and dx on the sampled tokens (their rows through inv_perm)
    sub_inv = inv_perm.reshape(T, k)[toks].reshape(-1)
    sub_rows = dlr[sub_inv]
    ident = np.arange(len(toks) * k, dtype=np.int32)
    check_router_stage(xs, C, idx[toks], dw[toks], ident, None, None,
                       OF.bf16_value_from_bits(dx_in[toks]), sub_rows,
                       bf16_values_host(dx_out)[toks], None, "router bwd V3 sampled tokens")
    # dC on sampled experts: each expert's rows in row order
    xv = OF.bf16_value_from_bits(x)
    dCh = host(dC).astype(np.float64)
    for e in list(rng.choice(E, 6, replace=False)) + [int(np.argmax(np.diff(offs))),
                                                       int(np.argmin(np.diff(offs)))]:
        r0, r1 = int(offs[e]), int(offs[e + 1])
        prod = dlr[r0:r1, None].astype(np.float64) * xv[perm_src[r0:r1].astype(np.int64)]
        bnd = (r1 - r0 + 1) * 2.0 ** -24 * np.abs(prod).sum(0)
        assert (np.abs(dCh[e] - prod.sum(0)) <= bnd).all(), e
    # every expert's rows are that expert's tokens in ascending order
    assert np.all(np.diff(offs) >= 0) and offs[-1] == T * k


def _logical(c, sc, nch):
    """chunk-major [cap, C, 128], [cap, C] -> [C, 128 nch], [C, nch]"""
    C = c.shape[1]
    return (np.ascontiguousarray(c[:nch].transpose(1, 0, 2)).reshape(C, nch * 128),
            np.ascontiguousarray(sc[:nch].T))


# The FP8 MFMA's error on one 128-term dot product, relative to the sum of
# |products|: at most 2^-15.6 over 10^6 random-code dot products, but up to
# 2^-13.3 on these weight-gradient operands (128x1 tiles of w * dy and of h:
# a wide dynamic range within one tile), so the wgrad stage allows 2^-12.
MFMA_REL_WGRAD = 2.0 ** -12
# the rescaled accumulator's roundings per chunk (two scale quotients, their
# product, the multiply, the MFMA's add) plus the final scaling
WGRAD_ROUNDINGS = 6


def _wgrad_bound(qY, sY, qA, sA, pref):
    S = OG.grouped_wgrad(np.asarray(qY) & 0x7F, sY, np.asarray(qA) & 0x7F, sA, pref)
    nch = np.diff(pref).astype(np.float64)[:, None, None]
    return (MFMA_REL_WGRAD + WGRAD_ROUNDINGS * (nch + 1) * 2.0 ** -24) * S


@pytest.mark.parametrize("name", ["tiny", "mid"])
def test_layer_backward_small(name):
    """Every stage against the oracle applied to the GPU's own inputs to that
    stage (bit-exact codes and copies, GEMM outputs within their derived
    bounds, elementwise steps within one bf16 ulp), then the end result
    against the oracle's independent chain."""
    cfg = synth.CONFIGS[name]
    T, k, H, I, G = cfg.T, cfg.k, cfg.H, cfg.I, cfg.G
    log(f"[layer bwd] {name}: T={T} H={H} E={cfg.E} I={I}")
    layer, C, b = build_layer(cfg)
    x = synth.gen_x(cfg)
    dy = synth.gen_dy(cfg)
    x_d = bf16_dev(x)
    layer.forward(x_d)
    bufs = layer.buffers(T)
    bb = layer.backward(bf16_dev(dy), x_d, keep_intermediates=True)
    torch.cuda.synchronize()
    wts = oracle_weights(cfg)
    fwd = OL.layer(x, C, b, wts, cfg.n_group, cfg.topk_group, k, I)
    mism = compare_routes(host(bufs.topk_idx), fwd["route"], name)
    assert len(mism) == 0, "routing differs (near-tie): the backward comparison needs equal routing"
    offs = host(bufs.offsets).astype(np.int64)
    perm_src, inv_perm = host(bufs.perm_src)[:cfg.R], host(bufs.inv_perm)[:T * k]
    qgu = [wts.gu(g) for g in range(G)]
    qdn = [wts.dn(g) for g in range(G)]
    dyv, xv = OF.bf16_value_from_bits(dy), OF.bf16_value_from_bits(x)
    # combine backward on the GPU's D
    cb = OBK.combine_backward(dyv, bf16_values_host(bufs.d), inv_perm, host(bufs.topk_w), T, k, 1)
    dD = bf16_values_host(bb.dD)
    assert np.array_equal(dD, cb["dD"])
    Dv = bf16_values_host(bufs.d)
    rows = inv_perm.reshape(T, k).astype(np.int64)
    wb = H * 2.0 ** -23 * np.stack([np.sum(np.abs(dyv * Dv[rows[:, j]]), axis=1) for j in range(k)], 1)
    assert (np.abs(host(bb.dw) - cb["dw"]) <= wb).all()
    # dgrad down on the GPU's quantised dD
    qd, sd = OQ.quant_1x128(dD)
    assert np.array_equal(host(bb.dDq), qd) and np.array_equal(host(bb.dDs), sd)
    dnT = [OG.transpose_blocks(q, s_) for q, s_ in qdn]
    ref = OG.to_bf16(OG.grouped_dgrad(qd, sd, [q for q, _ in qdn], [s_ for _, s_ in qdn], offs))
    bound = gemm_accumulation_bound(qd, sd, [q for q, _ in dnT], [s_ for _, s_ in dnT], offs, H)
    assert_within_one_bf16_ulp(bf16_values_host(bb.dh), ref, f"{name} dh", bound)
    # recomputed gate+up
    ref = OG.to_bf16(OG.grouped_gemm(fwd["xq"][perm_src], fwd["xs"][perm_src], [q for q, _ in qgu],
                                     [s_ for _, s_ in qgu], offs))
    bound = gemm_accumulation_bound(fwd["xq"][perm_src], fwd["xs"][perm_src], [q for q, _ in qgu],
                                    [s_ for _, s_ in qgu], offs, H)
    gu = bf16_values_host(bb.gu)
    assert_within_one_bf16_ulp(gu, ref, f"{name} gate+up recomputed", bound)
    # SwiGLU backward on the GPU's GU and dh
    r_dgu, r_h = OBK.swiglu_backward(gu, bf16_values_host(bb.dh), I)
    dgu, h = bf16_values_host(bb.dgu), bf16_values_host(bb.h)
    for got, r, what in ((dgu, r_dgu, "dGU"), (h, r_h, "h")):
        assert (np.abs(got - r) <= bf16_ulp(np.maximum(np.abs(got), np.abs(r))) + 1e-30).all(), what
    # dgrad gate+up on the GPU's quantised dGU, then the unpermute
    qg, sg = OQ.quant_1x128(dgu)
    assert np.array_equal(host(bb.dguq), qg) and np.array_equal(host(bb.dgus), sg)
    guT = [OG.transpose_blocks(q, s_) for q, s_ in qgu]
    ref = OG.to_bf16(OG.grouped_dgrad(qg, sg, [q for q, _ in qgu], [s_ for _, s_ in qgu], offs))
    bound = gemm_accumulation_bound(qg, sg, [q for q, _ in guT], [s_ for _, s_ in guT], offs, 2 * I)
    dxp = bf16_values_host(bb.dxp)
    assert_within_one_bf16_ulp(dxp, ref, f"{name} dX", bound)
    ref_dx, dx64 = OC.combine(dxp, inv_perm, np.ones((T, k), np.float32), T, k, dxp[T * k:T * k + T])
    acc = (k + 1) * 2.0 ** -23 * (np.abs(dxp[rows]).sum(1) + np.abs(dxp[T * k:T * k + T]))
    assert_within_one_bf16_ulp(bf16_values_host(bb.dx), ref_dx, f"{name} dx", acc)
    # weight gradients on the GPU's 128x1 operands (themselves bit-exact)
    pref = OQ.chunk_prefix(offs)
    nch = int(pref[-1])
    for (c_, s_, src, what) in ((bb.c_dD, bb.s_dD, dD, "dD"), (bb.c_h, bb.s_h, h, "h"),
                                (bb.c_dgu, bb.s_dgu, dgu, "dGU"), (bb.c_x, bb.s_x, xv[perm_src], "x")):
        qo, so = OQ.quant_128x1_grouped(src.astype(np.float32), offs)
        ql, sl = _logical(host(c_), host(s_), nch)
        assert np.array_equal(ql, qo) and np.array_equal(sl, so), what
    for (cy, sy, ca, sa, dW, what) in ((bb.c_dD, bb.s_dD, bb.c_h, bb.s_h, bb.dW_dn, "dW_dn"),
                                       (bb.c_dgu, bb.s_dgu, bb.c_x, bb.s_x, bb.dW_gu, "dW_gu")):
        qy, sy_ = _logical(host(cy), host(sy), nch)
        qa, sa_ = _logical(host(ca), host(sa), nch)
        ref = OG.grouped_wgrad(qy, sy_, qa, sa_, pref)
        got = host(dW).astype(np.float64)
        bnd = _wgrad_bound(qy, sy_, qa, sa_, pref) + 1e-30
        ratio = np.abs(got - ref) / bnd
        if not (ratio <= 1).all():
            g_, n_, k_ = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
            log(f"[layer bwd] {what}: {int((ratio > 1).sum())} elements over the bound; worst "
                f"ratio {ratio.max():.3e} at group {g_} ({int(pref[g_ + 1] - pref[g_])} chunks) "
                f"n {n_} k {k_}: got {got[g_, n_, k_]!r} ref {ref[g_, n_, k_]!r} bound {bnd[g_, n_, k_]!r}; "
                f"nonfinite got {int((~np.isfinite(got)).sum())}")
        assert (ratio <= 1).all(), what
    # the router: on the GPU's own dw, routing and expert-path dx
    offs_r = offs[:cfg.E + 1]
    check_router_stage(x, C, host(bufs.topk_idx).reshape(T, k), host(bb.dw), inv_perm,
                       perm_src, offs_r, bf16_values_host(bb.dx), host(bb.dlogit_rows)[:T * k],
                       bf16_values_host(bb.dx_total), host(bb.dC), f"{name} router")
    # end to end against the oracle's own chain: the two chains requantise
    # slightly different bf16 intermediates (GEMM accumulation order) to E4M3,
    # so codes next to a rounding midpoint differ (one code step is 1/16 of an
    # element); relative L2 within 5e-3
    ref = OBK.layer_backward(dy, fwd, wts, x, C, T, k, I)
    errs = dict(dx=rel_l2(bf16_values_host(bb.dx_total), ref["dx"]),
                dx_expert=rel_l2(bf16_values_host(bb.dx), ref["dx_expert"]),
                dw=rel_l2(host(bb.dw), ref["dw"]), dC=rel_l2(host(bb.dC), ref["dC"]),
                dW_gu=rel_l2(host(bb.dW_gu), ref["dW_gu"]), dW_dn=rel_l2(host(bb.dW_dn), ref["dW_dn"]))
    log(f"[layer bwd] {name}: end to end " + ", ".join(f"{k_} {v:.2e}" for k_, v in errs.items()))
    assert max(errs.values()) <= 5e-3, errs


def test_layer_empty_batch():
    """T = 0: the forward (with the bias update and the balance statistic)
    and the backward run as no-ops: counts zero, bias unchanged, weight and
    centroid gradients zero."""
    cfg = synth.TINY
    layer, C, b = build_layer(cfg)
    log("[layer] empty batch T=0")
    x = torch.empty((0, cfg.H), dtype=torch.bfloat16, device="cuda")
    bias0 = host(layer.bias).copy()
    y = layer.forward(x, update_bias=True)
    assert tuple(y.shape) == (0, cfg.H)
    bufs = layer.buffers(0)
    torch.cuda.synchronize()
    assert not host(bufs.counts).any() and np.array_equal(host(layer.bias), bias0)
    assert not host(bufs.offsets).any()
    for seq_len in (None, 16):
        if seq_len:
            layer.forward(x, seq_len=seq_len)
        bb = layer.backward(torch.empty((0, cfg.H), dtype=torch.bfloat16, device="cuda"), x,
                            seq_len=seq_len)
        torch.cuda.synchronize()
        assert not host(bb.dW_gu).any() and not host(bb.dW_dn).any() and not host(bb.dC).any()
        assert tuple(bb.dx_total.shape) == (0, cfg.H)


@pytest.mark.parametrize("T", [200, 2048])   # small-group fallback; the fused 256-row kernel
def test_layer_backward_keep_gu_mid(T):
    """forward(keep_gu=True): the fused gate+up kernel also writes its bf16
    gate/up outputs and the backward reads them.  They are bit-identical to
    the gate+up GEMM the backward would rerun, the layer's output equals the
    plain forward's, and the gradients stay within the oracle bars."""
    cfg = synth.MID.with_(T=T)
    k, I, G = cfg.k, cfg.I, cfg.G
    layer, C, b = build_layer(cfg)
    x = synth.gen_x(cfg)
    dy = synth.gen_dy(cfg)
    log(f"[layer bwd keep_gu] mid: T={T}")
    x_d = bf16_dev(x)
    y = bf16_values_host(layer.forward(x_d, keep_gu=True))
    bufs = layer.buffers(T)
    bb = layer.backward(bf16_dev(dy), x_d)
    torch.cuda.synchronize()
    again = torch.empty_like(bufs.hgu)
    M.grouped_fp8_gemm(bufs.xq, bufs.xs, bufs.perm_src, layer.w_gu, layer.w_gu_s, bufs.offsets, G,
                       cfg.R, 2 * I, cfg.H, again)
    torch.cuda.synchronize()
    assert torch.equal(again.view(torch.int16), bufs.hgu.view(torch.int16))
    # the layer's output is the fused kernel's, whether it keeps them or not
    y_plain = bf16_values_host(layer.forward(x_d))
    torch.cuda.synchronize()
    assert np.array_equal(y, y_plain)
    wts = oracle_weights(cfg)
    fwd = OL.layer(x, C, b, wts, cfg.n_group, cfg.topk_group, k, I)
    assert len(compare_routes(host(bufs.topk_idx), fwd["route"], "mid")) == 0
    assert rel_l2(y, fwd["y"]) <= 2e-3
    ref = OBK.layer_backward(dy, fwd, wts, x, C, T, k, I)
    errs = dict(dx=rel_l2(bf16_values_host(bb.dx_total), ref["dx"]), dw=rel_l2(host(bb.dw), ref["dw"]),
                dC=rel_l2(host(bb.dC), ref["dC"]), dW_gu=rel_l2(host(bb.dW_gu), ref["dW_gu"]),
                dW_dn=rel_l2(host(bb.dW_dn), ref["dW_dn"]))
    log(f"[layer bwd keep_gu] mid: end to end " + ", ".join(f"{k_} {v:.2e}" for k_, v in errs.items()))
    assert max(errs.values()) <= 5e-3, errs


def test_layer_backward_after_weight_update():
    """A weight update through the layer (requantize_from_fp32: 128x128
    requantisation of new fp32 master weights) after a forward and backward
    on the old weights: the next forward and backward equal those of a fresh
    layer built from the new weights, bit for bit (nothing derived from the
    old weights survives the update)."""
    cfg = synth.MID
    layer, C, b = build_layer(cfg)
    x = bf16_dev(synth.gen_x(cfg))
    dy = bf16_dev(synth.gen_dy(cfg))
    layer.forward(x)
    layer.backward(dy, x)                       # on the first weights
    torch.cuda.synchronize()
    seed = 5
    gu = torch.stack([torch.from_numpy(synth.gen_expert_weight(cfg, "gu", e, seed=seed))
                      for e in range(cfg.G)]).cuda()
    dn = torch.stack([torch.from_numpy(synth.gen_expert_weight(cfg, "dn", e, seed=seed))
                      for e in range(cfg.G)]).cuda()
    layer.requantize_from_fp32(gu, dn)
    y1 = bf16_values_host(layer.forward(x))
    bb1 = layer.backward(dy, x)
    out1 = [bf16_values_host(bb1.dx_total), host(bb1.dW_gu), host(bb1.dW_dn), host(bb1.dC)]
    fresh = M.MoELayer.from_fp32_experts(
        layer.shape, torch.from_numpy(C).cuda(), torch.from_numpy(b).cuda(),
        ((e, synth.gen_expert_weight(cfg, "gu", e, seed=seed)) for e in range(cfg.G)),
        ((e, synth.gen_expert_weight(cfg, "dn", e, seed=seed)) for e in range(cfg.G)))
    y2 = bf16_values_host(fresh.forward(x))
    bb2 = fresh.backward(dy, x)
    out2 = [bf16_values_host(bb2.dx_total), host(bb2.dW_gu), host(bb2.dW_dn), host(bb2.dC)]
    assert np.array_equal(y1, y2)
    for name, a, c in zip(("dx", "dW_gu", "dW_dn", "dC"), out1, out2):
        assert np.array_equal(a, c), name
    log("[update] forward and backward after requantize_from_fp32 equal a fresh layer's")
