"""Pins of the oracle router: brute force over group and expert subsets,
hand-traced tie cases, the special case without a group limit (plain top-k),
scalar-loop weights, and the invariants of the selection."""
import itertools
import math
import os

import numpy as np
import pytest

import synth
from conftest import GOLDEN
from oracle import route as RT


def _brute_force_token(sb, s, n_group, topk_group, k):
    """Exhaustive: best group subset by total group score, then best k-subset.

    Group score is the best pair sum inside the group.  Ties between subsets
    are broken toward the lexicographically smallest index tuple, which is
    the lower-index-wins rule.
    """
    E = len(sb)
    gs = E // n_group
    gscore = []
    for g in range(n_group):
        vals = sb[g * gs:(g + 1) * gs]
        gscore.append(max(vals[a] + vals[b] for a, b in itertools.combinations(range(gs), 2)))
    best_g = None
    for sub in itertools.combinations(range(n_group), topk_group):
        tot = sum(gscore[g] for g in sub)
        if best_g is None or tot > best_g[0]:
            best_g = (tot, sub)
    kept = [e for g in best_g[1] for e in range(g * gs, (g + 1) * gs)]
    best_e = None
    for sub in itertools.combinations(kept, k):
        tot = sum(sb[e] for e in sub)
        if best_e is None or tot > best_e[0]:
            best_e = (tot, sub)
    ids = sorted(best_e[1])
    den = sum(s[e] for e in ids)
    return ids, [s[e] / den for e in ids]


def _tiny_inputs(seed=0, T=64):
    cfg = synth.TINY
    x = synth.gen_x(cfg, seed=seed, T=T)
    c = synth.gen_centroids(cfg, seed=seed)
    b = synth.gen_bias(cfg, seed=seed)
    return cfg, x, c, b


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_tiny(seed):
    cfg, x, c, b = _tiny_inputs(seed)
    r = RT.route(x, c, b, cfg.n_group, cfg.topk_group, cfg.k)
    for t in range(cfg.T):
        ids, w = _brute_force_token(r["sb"][t], r["s"][t], cfg.n_group, cfg.topk_group, cfg.k)
        assert r["idx"][t].tolist() == ids
        np.testing.assert_allclose(r["w"][t], w, rtol=1e-14)


def test_brute_force_other_shapes():
    # 24 experts in 6 groups of 4, keep 3, top-5 (odd k, partial group use)
    cfg = synth.TINY.with_(E=24, n_group=6, topk_group=3, k=5)
    x = synth.gen_x(cfg, seed=3, T=40)
    c = synth.gen_centroids(cfg, seed=3) * 4
    b = synth.gen_bias(cfg, seed=3)
    r = RT.route(x, c, b, cfg.n_group, cfg.topk_group, cfg.k)
    for t in range(40):
        ids, w = _brute_force_token(r["sb"][t], r["s"][t], 6, 3, 5)
        assert r["idx"][t].tolist() == ids


def test_scores_scalar_loop():
    cfg, x, c, b = _tiny_inputs(0, T=4)
    r = RT.route(x, c, b, cfg.n_group, cfg.topk_group, cfg.k)
    xv = (x.astype(np.uint32) << 16).view(np.float32)
    for t in range(4):
        for e in range(cfg.E):
            logit = math.fsum(float(xv[t, h]) * float(c[e, h]) for h in range(cfg.H))
            sig = 1.0 / (1.0 + math.exp(-logit))
            assert abs(r["s"][t, e] - sig) < 1e-15
            assert abs(r["sb"][t, e] - (sig + float(b[e]))) < 1e-15


def _ties_rows():
    rows = []
    with open(os.path.join(GOLDEN, "route_ties.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            shape, biases, ids, ws, margin = [p.strip() for p in line.split("|")]
            E, ng, tg, k = map(int, shape.split())
            b = np.zeros(E, np.float32)
            if biases != "-":
                for item in biases.split(","):
                    e, v = item.split(":")
                    b[int(e)] = np.float32(float(v))
            rows.append((E, ng, tg, k, b, [int(i) for i in ids.split(",")],
                         [float(w) for w in ws.split(",")], float(margin)))
    return rows


@pytest.mark.parametrize("row", _ties_rows())
def test_hand_traced_ties(row):
    E, ng, tg, k, b, ids, ws, margin = row
    H = 256
    x = np.zeros((3, H), np.uint16)              # bf16 zeros -> every s = 1/2
    c = synth.gen_centroids(synth.TINY.with_(E=E, H=H))
    r = RT.route(x, c, b, ng, tg, k)
    for t in range(3):
        assert r["idx"][t].tolist() == ids
        assert r["w"][t].tolist() == ws
        assert r["margin"][t] == margin
    assert r["counts"].sum() == 3 * k


def test_no_group_limit_is_plain_topk():
    cfg = synth.MID
    x = synth.gen_x(cfg, T=64)
    c = synth.gen_centroids(cfg)
    b = synth.gen_bias(cfg)
    r = RT.route(x, c, b, cfg.n_group, cfg.n_group, cfg.k)   # keep every group
    s, sb = r["s"], r["sb"]
    for t in range(64):
        top = sorted(range(cfg.E), key=lambda e: (-sb[t, e], e))[:cfg.k]
        assert r["idx"][t].tolist() == sorted(top)
    r1 = RT.route(x, c, b, 1, 1, cfg.k)                      # one group of all experts
    assert np.array_equal(r1["idx"], r["idx"])


def test_invariants_v3_shape():
    cfg = synth.DECODE
    x = synth.gen_x(cfg, T=128)
    c = synth.gen_centroids(cfg)
    b = synth.gen_bias(cfg)
    r = RT.route(x, c, b, cfg.n_group, cfg.topk_group, cfg.k)
    idx = r["idx"]
    assert idx.shape == (128, 8)
    assert np.all(np.diff(idx, axis=1) > 0)                  # distinct, ascending
    assert np.all([len(set(row // 32)) <= 4 for row in idx])
    np.testing.assert_allclose(r["w"].sum(axis=1), 1.0, atol=1e-12)
    assert r["counts"].sum() == 128 * 8
    assert np.all(r["margin"] > 0)


def test_bias_selects_but_does_not_weight():
    cfg, x, c, b = _tiny_inputs(1, T=32)
    r0 = RT.route(x, c, np.zeros_like(b), cfg.n_group, cfg.topk_group, cfg.k)
    # pick, per token, a kept expert that was not chosen and push it with a
    # large bias inside its own group; it must then be chosen, and the weights
    # must still be the normalised unbiased scores of the chosen set
    for t in range(32):
        groups = set(r0["idx"][t] // 4)
        cand = [e for e in range(cfg.E) if e // 4 in groups and e not in r0["idx"][t]]
        e = cand[0]
        bb = np.zeros(cfg.E, np.float32)
        bb[e] = 5.0
        r1 = RT.route(x[t:t + 1], c, bb, cfg.n_group, cfg.topk_group, cfg.k)
        assert e in r1["idx"][0]
        ssel = r1["s"][0, r1["idx"][0]]
        np.testing.assert_allclose(r1["w"][0], ssel / ssel.sum(), rtol=1e-15)
        assert r1["w"][0].max() < 0.99     # a biased expert is not weighted by its bias


def _brute_force_margin(sb, n_group, topk_group, k):
    """The gap that decided one token's choice, from explicit sorts.

    Group gap: every group's score is its best pair sum (all pairs tried);
    the scores are sorted in descending order, and the gap is the
    topk_group-th minus the next one.  Expert gap: the groups kept are the
    topk_group best by (score descending, index ascending); their experts'
    biased scores are sorted in descending order and the gap is the k-th
    minus the next one.  A gap with no next element is inf.
    """
    E = len(sb)
    gs = E // n_group
    gscore = [max(float(sb[g * gs + a]) + float(sb[g * gs + b])
                  for a, b in itertools.combinations(range(gs), 2)) for g in range(n_group)]
    ranked = sorted(range(n_group), key=lambda g: (-gscore[g], g))
    if topk_group < n_group:
        ggap = gscore[ranked[topk_group - 1]] - gscore[ranked[topk_group]]
    else:
        ggap = math.inf
    kept = sorted(float(sb[g * gs + i]) for g in ranked[:topk_group] for i in range(gs))[::-1]
    egap = kept[k - 1] - kept[k] if k < len(kept) else math.inf
    return min(ggap, egap)


@pytest.mark.parametrize("shape", [(16, 4, 2, 4), (24, 6, 3, 5), (16, 4, 4, 4), (16, 4, 2, 8),
                                   (64, 8, 4, 8), (16, 1, 1, 3)])
def test_margin_brute_force(shape):
    """select()'s margin equals the brute-force gaps exactly on random scores
    (distinct values, so an off-by-one in either gap, or a group gap taken
    from the wrong pair, changes the number)."""
    E, ng, tg, k = shape
    cfg = synth.TINY.with_(E=E, n_group=ng, topk_group=tg, k=k)
    x = synth.gen_x(cfg, seed=E + k, T=48)
    c = synth.gen_centroids(cfg, seed=E + k) * 8
    b = synth.gen_bias(cfg, seed=E + k)
    r = RT.route(x, c, b, ng, tg, k)
    forced = tg == ng and k == E
    assert np.all(np.isfinite(r["margin"])) != forced
    for t in range(48):
        assert r["margin"][t] == _brute_force_margin(r["sb"][t], ng, tg, k), t


def test_margin_forced_choice_is_inf():
    """Every group kept and every expert chosen: nothing was decided."""
    cfg = synth.TINY.with_(E=8, n_group=2, topk_group=2, k=8)
    x = synth.gen_x(cfg, T=5)
    r = RT.route(x, synth.gen_centroids(cfg), synth.gen_bias(cfg), 2, 2, 8)
    assert np.all(np.isinf(r["margin"]))
    assert np.array_equal(r["idx"], np.tile(np.arange(8, dtype=np.int32), (5, 1)))
