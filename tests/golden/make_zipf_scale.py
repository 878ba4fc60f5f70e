"""Fit the per-expert centroid scale factors of the skewed-load workload and
write them to zipf_scale.txt (run once; the file is committed).

Workload recipe (no page defines one; this is the build's reading): router
centroids C ~ N(0, 0.02) as for the other V3-shape workloads, with expert
e's row multiplied by a factor a_e > 0.  The factors are chosen so that the
fraction of tokens that select expert e follows p_e = min(1, c * rank_e^-1.1)
with sum_e p_e = k (a Zipf(1.1) popularity over a random ranking of the
experts; the per-token cap of 1 is needed because a token selects an expert
at most once).  The fit takes fixed-point steps on log a_e on a calibration
batch that the measured runs never see:
    log a_e += 0.3 * (log p_e(target) - log p_e(achieved)),
with the step clipped to +-0.5 and a_e kept in [0.05, 20].  Routing is the
oracle's (sigmoid scores, zero bias, 4-of-8 groups, top-8).  Scaling a row
widens its zero-mean logit distribution, which raises how often the expert
wins, but a token picks an expert only when its logit is large and positive,
so popularities near 1 are out of reach; the achieved curve is recorded.

Usage: python tests/golden/make_zipf_scale.py [T_cal] [iterations]
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path[:0] = [ROOT]

import synth  # noqa: E402
from oracle import route as OR  # noqa: E402


def zipf_target(ranks: np.ndarray, k: int, s: float) -> np.ndarray:
    """p = min(1, c * rank^-s) with sum p = k (c by bisection)."""
    base = ranks.astype(np.float64) ** -s
    lo, hi = 0.0, float(k) / base.min()
    for _ in range(200):
        c = 0.5 * (lo + hi)
        if np.minimum(1.0, c * base).sum() < k:
            lo = c
        else:
            hi = c
    return np.minimum(1.0, 0.5 * (lo + hi) * base)


def main():
    T_cal = int(sys.argv[1]) if len(sys.argv) > 1 else 4096
    iters = int(sys.argv[2]) if len(sys.argv) > 2 else 40
    cfg = synth.SKEWED
    ranks = synth.zipf_ranks(cfg.E)
    target = zipf_target(ranks, cfg.k, synth.ZIPF_S)
    x = synth.gen_x(cfg, seed=synth.ZIPF_CAL_SEED, T=T_cal)
    b = np.zeros(cfg.E, np.float32)
    log_a = np.zeros(cfg.E)
    floor = 0.5 / T_cal
    for it in range(iters + 1):
        a = np.exp(log_a).astype(np.float32)
        r = OR.route(x, synth.gen_zipf_centroids(cfg, a), b, cfg.n_group, cfg.topk_group, cfg.k)
        p = r["counts"] / T_cal
        err = np.log(np.maximum(target, floor)) - np.log(np.maximum(p, floor))
        print(f"iter {it}: max/mean load {p.max() * cfg.E / cfg.k:.2f}, "
              f"mean |log p/target| {np.abs(err).mean():.3f}", flush=True)
        if it == iters:
            break
        log_a = np.clip(log_a + np.clip(0.3 * err, -0.5, 0.5), np.log(0.05), np.log(20.0))
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "zipf_scale.txt")
    with open(out, "w") as f:
        f.write("# Skewed-load workload: per-expert scale factors of the router centroids,\n"
                "# written by tests/golden/make_zipf_scale.py (oracle routing on a\n"
                f"# calibration batch: T={T_cal}, seed {synth.ZIPF_CAL_SEED}, {iters} fixed-point steps).\n"
                "# Target: fraction of tokens selecting expert e = min(1, c * rank^-1.1), sum = k = 8,\n"
                "# over a random ranking (synth.zipf_ranks).  Achieved: that fraction on the\n"
                "# calibration batch with these factors.\n"
                "# columns: expert scale rank target achieved\n")
        for e in range(cfg.E):
            f.write(f"{e} {float(a[e]):.9g} {int(ranks[e])} {target[e]:.6f} {p[e]:.6f}\n")
    print("wrote", out)


if __name__ == "__main__":
    main()
