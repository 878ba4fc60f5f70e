"""Whole-layer GPU parity against the oracle, through the C ABI.

* tiny and mid configs: every intermediate against the grouped oracle
  (indices, counts, permutation and activation codes bit-exact; GEMM outputs
  within the derived rounding bound; layer output rel L2 <= 2e-3);
* V3 shapes at T=128 (decode) and T=16384 (prefill), in the launch
  configuration the benchmark times: routing of every token against the
  FP64 oracle (near-ties logged); permutation maps and the activation codes
  and scales of every token bit-exact; every E4M3 code of h on the checked
  tokens against the exact gate/up sums; the layer output of all 128 decode
  tokens and of 256 sampled prefill tokens against the direct per-token
  oracle (rel L2 <= 2e-3);
* the skewed-load workload (T=8192, Zipf-scaled centroids, bias from 0):
  three steps on fresh batches with the bias update after each, against the
  oracle's own bias trajectory.
"""
import os
import time

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
from oracle import permute as OP
from oracle import quant as OQ
from oracle import route as OR
from oracle.formats import bf16_value_from_bits

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


THREADS = min(16, len(os.sched_getaffinity(0)))


@pytest.fixture(scope="module")
def v3_oracle_weights():
    """The oracle's own 128x128 quantisation of all 257 V3 experts (the decode,
    prefill and skewed workloads share the weights), cached for the module."""
    cfg = synth.DECODE
    wts = oracle_weights(cfg)
    t0 = time.time()
    for e0 in range(0, cfg.G, 32):
        wts.prefetch(range(e0, min(e0 + 32, cfg.G)), threads=THREADS)
        log(f"[layer] oracle quantised experts < {min(e0 + 32, cfg.G)} "
            f"({time.time() - t0:.0f} s, {THREADS} threads)")
    return wts


@pytest.mark.timeout(900)
def test_layer_v3_weights_quantised(v3_layer, v3_oracle_weights):
    """The GPU 128x128 quantiser's codes and scales of all 257 experts' gate/up
    and down weights equal the oracle's, byte for byte."""
    layer = v3_layer[0]
    for e in range(synth.DECODE.G):
        qg, sg = v3_oracle_weights.gu(e)
        qd, sd = v3_oracle_weights.dn(e)
        assert np.array_equal(host(layer.w_gu[e]), qg) and np.array_equal(host(layer.w_gu_s[e]), sg), e
        assert np.array_equal(host(layer.w_dn[e]), qd) and np.array_equal(host(layer.w_dn_s[e]), sd), e
    log(f"[layer] V3 weights of all {synth.DECODE.G} experts bit-exact")


def _slot_rows(inv_perm, tokens, T, k):
    """GPU rows of token t's slots (routed slots through inv_perm, then the
    shared row T*k + t), [n, k + 1]."""
    inv = inv_perm[:T * k].reshape(T, k)[tokens]
    return np.concatenate([inv, (T * k + np.asarray(tokens))[:, None]], axis=1)


def _accumulation_bounds(ref, idx, wts, cfg, threads):
    """Per (token, slot) bound on the GPU's deviation from the exact gate/up
    sums (gemm_accumulation_bound on the token's rows and the expert's
    weights), [n, k + 1, 2I]."""
    from concurrent.futures import ThreadPoolExecutor
    n, E, k = idx.shape[0], cfg.E, cfg.k
    qa, sa = ref["xq"], ref["xs"]

    def run(e):
        if e < E:
            rows, slots = np.nonzero(idx == e)
        else:
            rows, slots = np.arange(n), np.full(n, k)
        qB, sB = wts.gu(e)
        off = np.array([0, len(rows)], np.int64)
        return rows, slots, gemm_accumulation_bound(qa[rows], sa[rows], [qB], [sB], off, cfg.H)

    out = np.zeros((n, k + 1, 2 * cfg.I))
    experts = sorted(set(idx.ravel().tolist())) + [E]
    with ThreadPoolExecutor(threads) as ex:
        for i, (rows, slots, bnd) in enumerate(ex.map(run, experts)):
            out[rows, slots] = bnd
            if (i + 1) % 64 == 0:
                log(f"[layer] accumulation bounds: {i + 1} of {len(experts)} experts")
    return out


def _v3_check(v3_layer, wts, cfg, tokens, label):
    """The layer at V3 shapes in the launch configuration the benchmark times:
    routing of every token against the FP64 oracle (near-ties logged); the
    permutation maps bit-exact against the oracle's permutation of the GPU's
    routing (and of the oracle's, when they agree); the 1x128 codes and scales
    of every token bit-exact; on the given tokens every E4M3 code of h checked
    per element against the exact gate/up sums (a differing code must be a
    one-step flip at a rounding midpoint within the GEMM's bound), and the
    output's relative L2 over those tokens <= 2e-3 (per-token values logged)."""
    layer, C, b = v3_layer
    T, k, E, I = cfg.T, cfg.k, cfg.E, cfg.I
    log(f"[layer] {label} T={T}: forward")
    x = synth.gen_x(cfg)
    y = layer.forward(bf16_dev(x))
    got = bf16_values_host(y)
    bufs = layer.buffers(T)
    idx = host(bufs.topk_idx)
    ora = OR.route(x, C, b, cfg.n_group, cfg.topk_group, k)
    mism = compare_routes(idx, ora, f"{label}")
    cnt = host(bufs.counts)
    assert cnt.sum() == T * k and np.array_equal(cnt, np.bincount(idx.ravel(), minlength=E))
    off, ps, inv = host(bufs.offsets), host(bufs.perm_src)[:cfg.R], host(bufs.inv_perm)[:T * k]
    o_off, o_ps, o_inv = OP.permute(idx, E, 1)
    assert np.array_equal(off, o_off) and np.array_equal(ps, o_ps) and np.array_equal(inv, o_inv)
    if len(mism) == 0:
        r_off, r_ps, r_inv = OP.permute(ora["idx"], E, 1)
        assert np.array_equal(off, r_off) and np.array_equal(ps, r_ps) and np.array_equal(inv, r_inv)
        assert np.array_equal(cnt, ora["counts"])
    log(f"[layer] {label}: permutation maps ({cfg.R} rows) bit-exact")
    xq, xs = OQ.quant_1x128(bf16_value_from_bits(x).astype(np.float32))
    assert np.array_equal(host(bufs.xq), xq) and np.array_equal(host(bufs.xs), xs)
    log(f"[layer] {label}: 1x128 codes and scales of all {T} tokens bit-exact")

    tokens = np.array([t for t in tokens if t not in set(mism.tolist())], np.int64)
    t0 = time.time()
    # the oracle runs on slices of the tokens (every result is per token), so
    # that progress is logged while it works
    parts = []
    for i0 in range(0, len(tokens), 64):
        parts.append(OL.layer_tokens(x, C, b, wts, cfg.n_group, cfg.topk_group, k, I,
                                     tokens[i0:i0 + 64], keep=True, threads=THREADS))
        log(f"[layer] {label}: oracle on {min(i0 + 64, len(tokens))} of {len(tokens)} tokens "
            f"({time.time() - t0:.0f} s)")
    ref = {key: np.concatenate([np.atleast_1d(p_[key]) for p_ in parts]) for key in parts[0]}
    assert np.array_equal(ref["idx"], idx[tokens])
    log(f"[layer] {label}: oracle on {len(tokens)} tokens in {time.time() - t0:.0f} s")
    rows = _slot_rows(inv, tokens, T, k)
    rr = torch.from_numpy(rows.ravel().astype(np.int64)).cuda()
    hq = host(bufs.hq.index_select(0, rr))
    hs = host(bufs.hs.index_select(0, rr))
    d = bf16_values_host(bufs.d.index_select(0, rr)).reshape(len(tokens), k + 1, cfg.H)
    bound = _accumulation_bounds(ref, idx[tokens], wts, cfg, THREADS)
    log(f"[layer] {label}: accumulation bounds of the tokens' gate/up sums ({time.time() - t0:.0f} s)")
    nflip = check_fused_swiglu(hq, hs, ref["hgu"].reshape(-1, 2 * I), bound.reshape(-1, 2 * I), I,
                               f"{label} gate+up+SwiGLU")
    log(f"[layer] {label}: rel L2 of D over the tokens' {rows.size} rows = "
        f"{rel_l2(d, ref['D']):.3e}; h codes differing {nflip} of {hq.size}")
    per_tok = np.array([rel_l2(got[t], ref["y"][i]) for i, t in enumerate(tokens)])
    rel = rel_l2(got[tokens], ref["y"])
    log(f"[layer] {label}: per-token rel L2 median {np.median(per_tok):.2e}, max "
        f"{per_tok.max():.2e} (token {tokens[per_tok.argmax()]})")
    log(f"[layer] {label}: rel L2 of y over {len(tokens)} tokens vs oracle = {rel:.3e} "
        f"(bar {REL_L2_BAR})")
    assert rel <= REL_L2_BAR


def _sample(T, n, seed):
    rng = np.random.default_rng(seed)
    return sorted(set([0, T - 1] + rng.choice(T, n - 2, replace=False).tolist()))


@pytest.mark.timeout(1200)
def test_layer_v3_decode(v3_layer, v3_oracle_weights):
    """Decode batch: every one of the 128 tokens (the whole output tensor)."""
    _v3_check(v3_layer, v3_oracle_weights, synth.DECODE, np.arange(128), "v3-decode")


@pytest.mark.timeout(1200)
def test_layer_v3_prefill(v3_layer, v3_oracle_weights):
    """Prefill batch: 256 sampled tokens of 16384, everything else in full."""
    _v3_check(v3_layer, v3_oracle_weights, synth.PREFILL, _sample(16384, 256, 2), "v3-prefill")


@pytest.mark.timeout(600)
def test_layer_skewed_bias_steps(v3_layer, v3_oracle_weights):
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
            ref = OL.layer_tokens(x, C, b_used, v3_oracle_weights, cfg.n_group, cfg.topk_group,
                                  cfg.k, cfg.I, sample, threads=THREADS)
            rel = rel_l2(got[sample], ref["y"])
            log(f"[skewed] step 0: rel L2 of sampled y ({len(sample)} tokens) = {rel:.3e}")
            assert rel <= REL_L2_BAR


def test_layer_bias_save_resume(tmp_path):
    """Checkpoint/resume of the layer's only state, the fp32 selection bias
    (news.qq.com article, section 无额外损耗的负载均衡: the bias moves by
    gamma per step with the load): on the mid layer, 100 forward steps on
    fresh batches (seed 1000 + step) with the bias update after each, against
    50 steps, the bias saved to a file, a new layer built around the loaded
    bias, and 50 more steps - every step's bias and the last output bit for
    bit; and the trajectory against the oracle's (router + bias update in
    FP64 / fp32 on the same batches, from the oracle's own bias)."""
    cfg = synth.MID
    layer, C, b0 = build_layer(cfg)
    shape = layer.shape

    def run(lay, first, steps):
        traj, y = [], None
        for step in range(first, first + steps):
            x = synth.gen_x(cfg, seed=1000 + step)
            y = bf16_values_host(lay.forward(bf16_dev(x), update_bias=True))
            traj.append(host(lay.bias).copy())
        return traj, y

    def fresh(bias_np):
        return M.MoELayer(shape, layer.centroids, torch.from_numpy(bias_np).cuda(),
                          layer.w_gu, layer.w_gu_s, layer.w_dn, layer.w_dn_s)

    straight, y_straight = run(fresh(b0.copy()), 0, 100)
    first, _ = run(fresh(b0.copy()), 0, 50)
    np.save(tmp_path / "bias.npy", first[-1])
    resumed, y_resumed = run(fresh(np.load(tmp_path / "bias.npy")), 50, 50)
    for i, (a, b) in enumerate(zip(first + resumed, straight)):
        assert np.array_equal(a, b), f"step {i}"
    assert np.array_equal(y_resumed, y_straight)
    b_ora = b0.copy()
    n_near = 0
    for step in range(100):
        x = synth.gen_x(cfg, seed=1000 + step)
        ora = OR.route(x, C, b_ora, cfg.n_group, cfg.topk_group, cfg.k)
        n_near += int((ora["margin"] < 1e-6).sum())
        b_ora = OB.bias_update(ora["counts"], b_ora)
        if n_near == 0:
            assert np.array_equal(straight[step], b_ora), f"step {step} vs oracle"
    log(f"[state] 100 bias steps: resumed == straight; vs oracle bit-exact "
        f"({'all steps' if n_near == 0 else 'until the first near-tie'}); "
        f"bias range [{straight[-1].min():.4f}, {straight[-1].max():.4f}]")
