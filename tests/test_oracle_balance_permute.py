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
