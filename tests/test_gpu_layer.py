"""Whole-layer GPU parity against the oracle, through the C ABI.

* tiny and mid configs: every intermediate against the grouped oracle
  (indices, counts, permutation and activation codes bit-exact; GEMM outputs
  within the derived rounding bound; layer output rel L2 <= 2e-3);
* V3 shapes at T=128 (decode) and T=16384 (prefill), in the launch
  configuration the benchmark times: routing of every token against the
  FP64 oracle (near-ties logged), the GPU weight quantiser against the
  oracle's on the touched experts, and the layer output of sampled tokens
  against the direct per-token oracle (rel L2 <= 2e-3);
* the skewed-load workload (T=8192, Zipf-scaled centroids, bias from 0):
  three steps on fresh batches with the bias update after each, against the
  oracle's own bias trajectory.
"""
import numpy as np
import pytest
import torch

import synth
import fp8_block_scaled_bias_amd as M
from gpu_common import bf16_dev, bf16_values_host, host, log, rel_l2, compare_routes
from test_gpu_kernels import check_fused_swiglu, gemm_accumulation_bound
from oracle import balance as OB
from oracle import gemm as OG
from oracle import layer as OL
from oracle import route as OR

pytestmark = pytest.mark.gpu

REL_L2_BAR = 2e-3


def shape_of(cfg):
    return M.LayerShape(cfg.H, cfg.E, cfg.n_group, cfg.topk_group, cfg.k, cfg.I, cfg.n_shared)


def build_layer(cfg):
    C = synth.gen_centroids(cfg)
    b = synth.gen_bias(cfg)
    layer = M.MoELayer.from_fp32_experts(
        shape_of(cfg), torch.from_numpy(C).cuda(), torch.from_numpy(b).cuda(),
        synth.gen_all_expert_weights(cfg, "gu"), synth.gen_all_expert_weights(cfg, "dn"))
    return layer, C, b


def oracle_weights(cfg):
    return OL.ExpertWeights(lambda e: synth.gen_expert_weight(cfg, "gu", e),
                            lambda e: synth.gen_expert_weight(cfg, "dn", e))


@pytest.mark.parametrize("name", ["tiny", "mid"])
def test_layer_full_small(name):
    cfg = synth.CONFIGS[name]
    log(f"[layer] {name}: T={cfg.T} H={cfg.H} E={cfg.E} I={cfg.I}")
    layer, C, b = build_layer(cfg)
    x = synth.gen_x(cfg)
    y = layer.forward(bf16_dev(x))
    got = bf16_values_host(y)
    bufs = layer.buffers(cfg.T)
    ref = OL.layer(x, C, b, oracle_weights(cfg), cfg.n_group, cfg.topk_group, cfg.k, cfg.I)
    mism = compare_routes(host(bufs.topk_idx), ref["route"], name)
    assert np.array_equal(host(bufs.xq), ref["xq"]) and np.array_equal(host(bufs.xs), ref["xs"])
    if len(mism) == 0:
        assert np.array_equal(host(bufs.counts), ref["route"]["counts"])
        assert np.array_equal(host(bufs.offsets), ref["offsets"])
        assert np.array_equal(host(bufs.perm_src)[:cfg.R], ref["perm_src"])
        assert np.array_equal(host(bufs.inv_perm)[:cfg.T * cfg.k], ref["inv_perm"])
        A, sA = ref["xq"][ref["perm_src"]], ref["xs"][ref["perm_src"]]
        wts = oracle_weights(cfg)
        qB = [wts.gu(g)[0] for g in range(cfg.G)]
        sB = [wts.gu(g)[1] for g in range(cfg.G)]
        bound = gemm_accumulation_bound(A, sA, qB, sB, ref["offsets"], cfg.H)
        check_fused_swiglu(host(bufs.hq), host(bufs.hs), ref["Hgu"], bound, cfg.I,
                           f"{name} fused gate+up")
    keep = np.setdiff1d(np.arange(cfg.T), mism)
    rel = rel_l2(got[keep], ref["y"][keep])
    log(f"[layer] {name}: rel L2 of y vs oracle = {rel:.3e} (bar {REL_L2_BAR})")
    assert rel <= REL_L2_BAR
    # determinism: a second forward is bit-identical
    y2 = bf16_values_host(layer.forward(bf16_dev(x)))
    assert np.array_equal(y2, got)


def test_layer_collapsed_routing():
    """Degenerate routing: every token identical, so all T tokens choose the
    same 8 experts (8 groups of T rows next to the shared group of T rows,
    56 empty groups), at T=2048 on the mid layer: the 256x256-tile kernel
    takes gate+up.  Output against the oracle, counts exact."""
    cfg = synth.MID.with_(T=2048)
    T = cfg.T
    layer, C, b = build_layer(cfg)
    x = np.repeat(synth.gen_x(cfg, T=1), T, axis=0)
    log(f"[layer] collapsed routing: T={T}, every token the same")
    got = bf16_values_host(layer.forward(bf16_dev(x)))
    bufs = layer.buffers(T)
    ref = OL.layer(x, C, b, oracle_weights(cfg), cfg.n_group, cfg.topk_group, cfg.k, cfg.I)
    assert len(compare_routes(host(bufs.topk_idx), ref["route"], "collapsed")) == 0
    cnt = host(bufs.counts)
    assert sorted(cnt.tolist())[-cfg.k:] == [T] * cfg.k and (cnt > 0).sum() == cfg.k
    assert np.array_equal(host(bufs.offsets), ref["offsets"])
    rel = rel_l2(got, ref["y"])
    log(f"[layer] collapsed: rel L2 of y vs oracle = {rel:.3e}")
    assert rel <= REL_L2_BAR
    assert np.array_equal(got, np.repeat(got[:1], T, axis=0))   # identical tokens, identical rows


@pytest.fixture(scope="module")
def v3_layer():
    cfg = synth.DECODE
    log("[layer] building V3-shape weights (257 experts, GPU 128x128 quantiser)")
    layer, C, b = build_layer(cfg)
    return layer, C, b


def _v3_check(v3_layer, cfg, sample):
    layer, C, b = v3_layer
    log(f"[layer] v3 T={cfg.T}: forward")
    x = synth.gen_x(cfg)
    y = layer.forward(bf16_dev(x))
    got = bf16_values_host(y)
    bufs = layer.buffers(cfg.T)
    idx = host(bufs.topk_idx)
    ora = OR.route(x, C, b, cfg.n_group, cfg.topk_group, cfg.k)
    mism = compare_routes(idx, ora, f"v3-T{cfg.T}")
    cnt = host(bufs.counts)
    assert cnt.sum() == cfg.T * cfg.k and np.array_equal(cnt, np.bincount(idx.ravel(), minlength=cfg.E))
    off = host(bufs.offsets)
    assert off[-1] == cfg.R and np.array_equal(np.diff(off)[:cfg.E], cnt)
    sample = [t for t in sample if t not in set(mism.tolist())]
    wts = oracle_weights(cfg)
    touched = set(ora["idx"][sample].ravel().tolist()) | {cfg.E}
    log(f"[layer] v3 T={cfg.T}: oracle on tokens {sample} ({len(touched)} experts)")
    wts.prefetch(touched)
    for e in sorted(touched)[:3]:
        qg, sg = wts.gu(e)
        assert np.array_equal(host(layer.w_gu[e]), qg) and np.array_equal(host(layer.w_gu_s[e]), sg)
        qd, sd = wts.dn(e)
        assert np.array_equal(host(layer.w_dn[e]), qd) and np.array_equal(host(layer.w_dn_s[e]), sd)
    ref = OL.layer_tokens(x, C, b, wts, cfg.n_group, cfg.topk_group, cfg.k, cfg.I, sample)
    per_tok = [rel_l2(got[t], ref["y"][i]) for i, t in enumerate(sample)]
    log(f"[layer] v3 T={cfg.T}: per-token rel L2 " + " ".join(f"{v:.2e}" for v in per_tok))
    rel = rel_l2(got[sample], ref["y"])
    log(f"[layer] v3 T={cfg.T}: rel L2 of sampled y ({len(sample)} tokens) vs oracle = "
        f"{rel:.3e} (bar {REL_L2_BAR})")
    assert rel <= REL_L2_BAR


def _sample(T, n, seed):
    rng = np.random.default_rng(seed)
    return sorted(set([0, T - 1] + rng.choice(T, n - 2, replace=False).tolist()))


def test_layer_v3_decode(v3_layer):
    _v3_check(v3_layer, synth.DECODE, _sample(128, 16, 1))


def test_layer_v3_prefill(v3_layer):
    _v3_check(v3_layer, synth.PREFILL, _sample(16384, 16, 2))


def test_layer_skewed_bias_steps(v3_layer):
    """Skewed-load workload: 3 steps, each on a fresh batch (seed 1000 + step)
    and followed by the bias update (news.qq.com article, section 无额外损耗的
    负载均衡: bias -/+ gamma for over/under-loaded experts).  Per step: routing
    of all 8192 tokens against the oracle run with the oracle's own bias
    trajectory (near-ties logged), counts exact, the updated bias bit-exact;
    at step 0 also the layer output of sampled tokens (rel L2 <= 2e-3)."""
    base = v3_layer[0]
    cfg = synth.SKEWED
    C = synth.gen_zipf_centroids(cfg)
    layer = M.MoELayer(base.shape, torch.from_numpy(C).cuda(),
                       torch.zeros(cfg.E, dtype=torch.float32, device="cuda"),
                       base.w_gu, base.w_gu_s, base.w_dn, base.w_dn_s)
    b_ora = np.zeros(cfg.E, np.float32)
    mean = cfg.T * cfg.k / cfg.E
    for step in range(3):
        log(f"[skewed] step {step}: forward")
        x = synth.gen_x(cfg, seed=synth.ZIPF_STEP_SEED0 + step)
        b_used = b_ora.copy()
        y = layer.forward(bf16_dev(x), update_bias=True)
        got = bf16_values_host(y)
        bufs = layer.buffers(cfg.T)
        ora = OR.route(x, C, b_used, cfg.n_group, cfg.topk_group, cfg.k)
        mism = compare_routes(host(bufs.topk_idx), ora, f"skewed step {step}")
        cnt = host(bufs.counts)
        log(f"[skewed] step {step}: max/mean load {cnt.max() / mean:.2f}")
        if len(mism) == 0:
            assert np.array_equal(cnt, ora["counts"])
        # the update follows the counts the GPU routed (equal unless a near-tie moved one)
        b_ora = OB.bias_update(cnt, b_ora)
        assert np.array_equal(host(layer.bias), b_ora)
        if step == 0:
            sample = [t for t in _sample(cfg.T, 8, 3) if t not in set(mism.tolist())]
            wts = oracle_weights(cfg)
            ref = OL.layer_tokens(x, C, b_used, wts, cfg.n_group, cfg.topk_group, cfg.k, cfg.I,
                                  sample)
            rel = rel_l2(got[sample], ref["y"])
            log(f"[skewed] step 0: rel L2 of sampled y ({len(sample)} tokens) = {rel:.3e}")
            assert rel <= REL_L2_BAR
