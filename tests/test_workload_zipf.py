"""The stored fit of the skewed-load workload (tests/golden/zipf_scale.txt,
written by tests/golden/make_zipf_scale.py with the oracle router).

Checks the file against its own recipe: 256 rows, scale factors inside the
fit's clamp, the ranking equal to synth.zipf_ranks, the target curve equal to
min(1, c * rank^-1.1) with sum 8, achieved fractions summing to 8 (each token
picks 8 experts) and falling with rank; and that the oracle router, given
these factors, produces a skewed load on tokens the fit never saw.
"""
import os
import sys

import numpy as np

import synth
from oracle import route as OR

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden"))
import make_zipf_scale  # noqa: E402


def _rows():
    rows = [l.split() for l in open(synth.ZIPF_SCALE_FILE) if l.strip() and not l.startswith("#")]
    return np.array([[float(v) for v in r] for r in rows])


def test_zipf_file_matches_recipe():
    r = _rows()
    E = synth.SKEWED.E
    assert r.shape == (E, 5)
    assert np.array_equal(r[:, 0], np.arange(E))
    scale = synth.load_zipf_scale()
    assert np.all(scale >= 0.05 * (1 - 1e-6)) and np.all(scale <= 20 * (1 + 1e-6))
    ranks = synth.zipf_ranks(E)
    assert np.array_equal(r[:, 2].astype(np.int64), ranks)
    target = make_zipf_scale.zipf_target(ranks, synth.SKEWED.k, synth.ZIPF_S)
    assert abs(target.sum() - synth.SKEWED.k) < 1e-6
    assert np.allclose(r[:, 3], target, atol=1e-6)
    assert abs(r[:, 4].sum() - synth.SKEWED.k) < 1e-3
    # achieved popularity falls with rank (Spearman correlation of -rank)
    order = np.argsort(np.argsort(-r[:, 4]))
    rho = np.corrcoef(order, ranks)[0, 1]
    assert rho > 0.9, rho


def test_zipf_centroids_give_skewed_load():
    cfg = synth.SKEWED
    x = synth.gen_x(cfg, seed=synth.ZIPF_STEP_SEED0, T=512)
    C = synth.gen_zipf_centroids(cfg)
    ranks = synth.zipf_ranks(cfg.E)
    r = OR.route(x, C, np.zeros(cfg.E, np.float32), cfg.n_group, cfg.topk_group, cfg.k)
    load = r["counts"] / (512 * cfg.k / cfg.E)
    assert load.max() > 8.0                          # a uniform router stays near 1
    top = np.argsort(ranks)[:16]
    assert load[top].mean() > 4.0 * load.mean()
