"""Pins of the oracle's bias update (closed forms of the sign rule) and of the
dispatch permutation (brute-force loop and bijection invariants)."""
import numpy as np
import pytest

from oracle import balance as BL
from oracle import permute as PM


def test_bias_update_closed_form():
    counts = np.array([5, 3, 4, 4, 0, 8], np.int32)     # total 24, mean 4
    b = np.array([0.0, 0.5, -0.25, 1.0, 0.0, -1.0], np.float32)
    g = np.float32(0.001)
    nb = BL.bias_update(counts, b, 0.001)
    exp = np.array([b[0] - g, b[1] + g, b[2], b[3], b[4] + g, b[5] - g], np.float32)
    assert np.array_equal(nb, exp)
    assert nb.dtype == np.float32


def test_bias_update_balanced_is_noop_and_sum_rule():
    b = np.random.default_rng(0).uniform(-0.01, 0.01, 256).astype(np.float32)
    assert np.array_equal(BL.bias_update(np.full(256, 32, np.int32), b), b)
    counts = np.random.default_rng(1).multinomial(256 * 8 * 16, np.full(256, 1 / 256)).astype(np.int32)
    nb = BL.bias_update(counts, np.zeros(256, np.float32))
    mean = counts.sum() / 256
    n_over = int((counts > mean).sum())
    n_under = int((counts < mean).sum())
    assert np.isclose(nb.astype(np.float64).sum(), 0.001 * (n_under - n_over), atol=1e-9)
    assert np.all((nb > 0) == (counts < mean)) and np.all((nb < 0) == (counts > mean))


def test_bias_update_uses_exact_integer_mean():
    # total 7 over 3 experts: mean 7/3 is not an integer; 2 < 7/3 < 3
    nb = BL.bias_update(np.array([2, 2, 3], np.int32), np.zeros(3, np.float32))
    assert nb.tolist() == [np.float32(0.001), np.float32(0.001), -np.float32(0.001)]


def _brute_permute(idx, E):
    T, k = idx.shape
    rows = []
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if idx[t, j] == e:
                    rows.append((t, j))
    perm_src = [t for t, _ in rows] + list(range(T))
    inv = np.empty(T * k, np.int64)
    for r, (t, j) in enumerate(rows):
        inv[t * k + j] = r
    return perm_src, inv


@pytest.mark.parametrize("T,k,E", [(1, 1, 4), (7, 3, 5), (50, 4, 16), (33, 8, 64)])
def test_permute_brute_force(T, k, E):
    rng = np.random.default_rng(T * 100 + E)
    idx = np.stack([np.sort(rng.choice(E, k, replace=False)) for _ in range(T)]).astype(np.int32)
    off, ps, inv = PM.permute(idx, E, 1)
    bps, binv = _brute_permute(idx, E)
    assert ps.tolist() == bps
    assert inv.tolist() == binv.tolist()
    counts = np.bincount(idx.ravel(), minlength=E)
    assert off.tolist() == [0] + list(np.cumsum(list(counts) + [T]))
    # bijection and consistency
    assert sorted(inv.tolist()) == list(range(T * k))
    for t in range(T):
        for j in range(k):
            r = inv[t * k + j]
            assert ps[r] == t and off[idx[t, j]] <= r < off[idx[t, j] + 1]


def test_permute_empty_experts_and_no_shared():
    idx = np.array([[3, 3], [3, 3]], np.int32)          # every row in expert 3
    off, ps, inv = PM.permute(idx, 6, 0)
    assert off.tolist() == [0, 0, 0, 0, 4, 4, 4]
    assert ps.tolist() == [0, 0, 1, 1] and inv.tolist() == [0, 1, 2, 3]


# ---- sequence-wise balance statistic ----------------------------------------

def _scores_and_choice(T, E, k, seed):
    rng = np.random.default_rng(seed)
    s = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, E))))
    idx = np.sort(np.stack([rng.choice(E, k, replace=False) for _ in range(T)]), 1)
    return s, idx


def test_seq_balance_python_loop():
    """Per sequence, expert by expert, in plain loops."""
    T, E, k, L, alpha = 11, 8, 3, 4, 0.25
    s, idx = _scores_and_choice(T, E, k, 3)
    st = BL.seq_balance(s, idx, L, alpha)
    starts = list(range(0, T, L))
    assert st["loss"].shape == (len(starts),)
    for b, t0 in enumerate(starts):
        toks = range(t0, min(T, t0 + L))
        n = len(toks)
        tot = 0.0
        for e in range(E):
            cnt = sum(1 for t in toks for j in range(k) if idx[t, j] == e)
            pe = sum(s[t, e] / sum(s[t, i] for i in range(E)) for t in toks) / n
            fe = E * cnt / (k * n)
            assert st["f"][b, e] == pytest.approx(fe, rel=1e-15)
            assert st["P"][b, e] == pytest.approx(pe, rel=1e-13)
            tot += fe * pe
        assert st["loss"][b] == pytest.approx(alpha * tot, rel=1e-13)


def test_seq_balance_closed_forms():
    T, E, k, L = 24, 16, 4, 8
    _, idx = _scores_and_choice(T, E, k, 5)
    # equal scores: P = 1/E and sum f = E, so the loss is alpha whatever the choice
    st = BL.seq_balance(np.full((T, E), 0.37), idx, L, 1e-4)
    np.testing.assert_allclose(st["loss"], 1e-4, rtol=1e-14)
    np.testing.assert_allclose(st["f"].sum(1), E, rtol=1e-14)
    # every token picks the same k experts with score a, the others score c:
    # loss = alpha E a / (k a + (E - k) c)
    a, c = 0.9, 0.2
    chosen = np.array([1, 5, 6, 11])
    s = np.full((T, E), c)
    s[:, chosen] = a
    st = BL.seq_balance(s, np.tile(chosen, (T, 1)), L, 1.0)
    np.testing.assert_allclose(st["loss"], E * a / (k * a + (E - k) * c), rtol=1e-14)
    assert not st["f"][:, np.setdiff1d(np.arange(E), chosen)].any()


def test_seq_balance_invariances():
    T, E, k, L = 30, 16, 4, 8
    s, idx = _scores_and_choice(T, E, k, 9)
    st = BL.seq_balance(s, idx, L)
    # tokens reordered inside each sequence: same statistic
    perm = np.concatenate([np.random.default_rng(1).permutation(np.arange(t0, min(T, t0 + L)))
                           for t0 in range(0, T, L)])
    st2 = BL.seq_balance(s[perm], idx[perm], L)
    for key in ("f", "P", "loss"):
        np.testing.assert_allclose(st2[key], st[key], rtol=1e-13)
    # the ragged last sequence (6 tokens) equals that sequence on its own
    last = BL.seq_balance(s[24:], idx[24:], 6)
    np.testing.assert_allclose(st["loss"][-1], last["loss"][0], rtol=1e-14)
    # scores scaled per token: s' and so the statistic are unchanged
    st3 = BL.seq_balance(s * np.linspace(0.5, 2.0, T)[:, None], idx, L)
    np.testing.assert_allclose(st3["loss"], st["loss"], rtol=1e-13)


def test_seq_balance_grad_is_the_derivative():
    """Central differences of the summed loss in each logit, selection fixed."""
    T, E, k, L = 10, 8, 2, 4
    rng = np.random.default_rng(17)
    logit = rng.standard_normal((T, E))
    idx = np.sort(np.stack([rng.choice(E, k, replace=False) for _ in range(T)]), 1)
    sig = lambda z: 1.0 / (1.0 + np.exp(-z))
    g = BL.seq_balance_grad_logits(sig(logit), idx, L, 0.5)
    eps = 1e-6
    for (t, e) in [(0, 0), (3, 5), (9, 7), (8, 2)]:
        lp, lm = logit.copy(), logit.copy()
        lp[t, e] += eps
        lm[t, e] -= eps
        fd = (BL.seq_balance(sig(lp), idx, L, 0.5)["loss"].sum()
              - BL.seq_balance(sig(lm), idx, L, 0.5)["loss"].sum()) / (2 * eps)
        assert abs(fd - g[t, e]) < 1e-9, (t, e, fd, g[t, e])


def _bias_steps(b, steps, first):
    """Route a fresh tiny batch (seed 1000 + step) with bias b, then update b
    from that batch's counts; returns the bias after each step."""
    import synth
    from oracle import route as RT
    cfg = synth.TINY
    c = synth.gen_centroids(cfg)
    out = []
    for step in range(first, first + steps):
        x = synth.gen_x(cfg, seed=1000 + step)
        r = RT.route(x, c, b, cfg.n_group, cfg.topk_group, cfg.k)
        b = BL.bias_update(r["counts"], b)
        out.append(b)
    return out


def test_bias_save_resume_equals_straight_run(tmp_path):
    """The layer's only state is the fp32 bias: 50 steps, save it to a file,
    load it into a fresh run, 50 more steps - the same trajectory, bit for
    bit, as 100 steps without the break."""
    b0 = np.zeros(16, np.float32)
    straight = _bias_steps(b0, 100, 0)
    first = _bias_steps(b0, 50, 0)
    np.save(tmp_path / "bias.npy", first[-1])
    resumed = _bias_steps(np.load(tmp_path / "bias.npy"), 50, 50)
    assert all(np.array_equal(a, b) for a, b in zip(first + resumed, straight))
    assert straight[-1].dtype == np.float32
    assert not np.array_equal(straight[49], straight[99])   # the bias did move
