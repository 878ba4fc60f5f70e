"""Pins of SwiGLU (closed-form values), combine (one-hot and uniform cases),
and the whole layer: grouped form against the direct per-token form."""
import math

import numpy as np
import pytest

import synth
from oracle import combine as CB
from oracle import layer as LY
from oracle import swiglu as SW
from oracle import formats as F


def test_silu_closed_forms():
    g = np.array([0.0, 1.0, -1.0, 20.0, -20.0, 2.5], np.float32)
    u = np.array([3.0, 1.0, 1.0, 1.0, 1.0, -2.0], np.float32)
    h = SW.silu_mul_fp32(g, u)
    exact = [x * (1.0 / (1.0 + math.exp(-x))) * y for x, y in zip(g.tolist(), u.tolist())]
    assert h[0] == 0.0
    np.testing.assert_allclose(h, exact, rtol=3e-7)
    np.testing.assert_allclose(h[1], 0.7310585786300049, rtol=2e-7)   # silu(1) = 1/(1+e^-1)


def test_swiglu_quant_zero_up_gives_zero_tile():
    I = 256
    hgu = np.zeros((2, 2 * I))
    hgu[:, :I] = np.random.default_rng(0).standard_normal((2, I))
    q, s, h = SW.swiglu_quant(F.bf16_round(hgu), I)
    assert np.all(h == 0) and np.all(s == 1.0)
    assert np.all((q == 0) | (q == 0x80))


def test_swiglu_uses_gate_then_up_halves():
    I = 128
    rng = np.random.default_rng(1)
    g = F.bf16_round(rng.standard_normal((3, I)))
    u = F.bf16_round(rng.standard_normal((3, I)))
    q, s, h = SW.swiglu_quant(np.concatenate([g, u], axis=1), I)
    q2, s2, h2 = SW.swiglu_quant(np.concatenate([u, g], axis=1), I)
    assert np.array_equal(h, SW.silu_mul_fp32(g, u))
    assert not np.array_equal(h, h2)


def test_combine_one_hot_and_uniform():
    T, k, H = 4, 3, 256
    rng = np.random.default_rng(2)
    D = F.bf16_round(rng.standard_normal((T * k + T, H)))
    inv = rng.permutation(T * k).astype(np.int32)
    w = np.zeros((T, k), np.float32)
    w[:, 1] = 1.0
    y, _ = CB.combine(D, inv, w, T, k, None)
    assert np.array_equal(y, D[inv.reshape(T, k)[:, 1]])
    Dsame = np.tile(D[:1], (T * k + T, 1))
    wu = np.full((T, k), np.float32(0.25))
    wu[:, 0] = 0.5
    y2, y64 = CB.combine(Dsame, inv, wu, T, k, Dsame[T * k:])
    np.testing.assert_array_equal(y64, 2.0 * Dsame[:T])


def _weights(cfg):
    return LY.ExpertWeights(lambda e: synth.gen_expert_weight(cfg, "gu", e),
                            lambda e: synth.gen_expert_weight(cfg, "dn", e))


def test_layer_grouped_equals_direct_per_token_tiny():
    cfg = synth.TINY
    x = synth.gen_x(cfg)
    c = synth.gen_centroids(cfg)
    b = synth.gen_bias(cfg)
    wts = _weights(cfg)
    out = LY.layer(x, c, b, wts, cfg.n_group, cfg.topk_group, cfg.k, cfg.I)
    direct = LY.layer_tokens(x, c, b, wts, cfg.n_group, cfg.topk_group, cfg.k, cfg.I,
                             np.arange(cfg.T))
    assert np.array_equal(out["route"]["idx"], direct["idx"])
    assert np.array_equal(out["y64"], direct["y64"])
    assert np.array_equal(out["y"], direct["y"])
    # kept per-slot values (the form the full-size GPU checks read) are the
    # grouped form's rows, and a thread pool changes nothing
    kept = LY.layer_tokens(x, c, b, wts, cfg.n_group, cfg.topk_group, cfg.k, cfg.I,
                           np.arange(cfg.T), keep=True, threads=4)
    assert np.array_equal(kept["y"], direct["y"])
    inv = out["inv_perm"].reshape(cfg.T, cfg.k)
    for t in range(cfg.T):
        rows = list(inv[t]) + [cfg.T * cfg.k + t]
        assert np.array_equal(kept["hgu"][t], out["Hgu"][rows])
        assert np.array_equal(kept["D"][t], out["D"][rows])
    assert np.array_equal(kept["xq"], out["xq"]) and np.array_equal(kept["xs"], out["xs"])
    # the layer output is not trivially small or dominated by the shared expert
    ys = out["D"][cfg.T * cfg.k:]
    assert np.linalg.norm(out["y64"] - ys) > 0.3 * np.linalg.norm(out["y64"])


def test_layer_against_float64_reference_tiny():
    # Without any FP8/bf16 storage points the layer is plain SwiGLU experts on
    # the unquantised weights; the quantised layer must stay close to it.
    cfg = synth.TINY
    x = synth.gen_x(cfg)
    c = synth.gen_centroids(cfg)
    b = synth.gen_bias(cfg)
    wts = _weights(cfg)
    out = LY.layer(x, c, b, wts, cfg.n_group, cfg.topk_group, cfg.k, cfg.I)
    xv = F.bf16_value_from_bits(x)
    ref = np.zeros_like(out["y64"])
    idx, w = out["route"]["idx"], out["route"]["w"]
    def ffn(e, row):
        wg = synth.gen_expert_weight(cfg, "gu", e).astype(np.float64)
        wd = synth.gen_expert_weight(cfg, "dn", e).astype(np.float64)
        hg = wg @ row
        g, u = hg[:cfg.I], hg[cfg.I:]
        return wd @ (g / (1 + np.exp(-g)) * u)
    for t in range(cfg.T):
        for j in range(cfg.k):
            ref[t] += w[t, j] * ffn(int(idx[t, j]), xv[t])
        ref[t] += ffn(cfg.E, xv[t])
    rel = np.linalg.norm(out["y64"] - ref) / np.linalg.norm(ref)
    assert rel < 0.08, rel          # FP8 activations+weights: a few percent
