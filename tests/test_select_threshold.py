"""Host check of the selection rule the router's select kernel applies (its
top-k among the kept experts), written out on the CPU: a threshold on the
order-preserving 32-bit keys of the biased scores, built bit by bit from
counts (from the top bit, or from below the bits every kept key shares),
stopping as soon as exactly k keys reach it; when it ends on a key
shared by several slots, every slot above it is taken and, of the equal ones,
the lowest expert ids.  Compared with a stable sort (score descending, id
ascending) on random scores, on scores forced into ties, and with dropped
groups.  It checks the rule, not the kernel (the GPU routing tests do that).
"""
import numpy as np


def _ord_keys(sb, kept):
    u = sb.astype(np.float32).view(np.uint32).copy()
    u[sb == 0.0] = 0                      # -0 as +0
    neg = (u & 0x80000000) != 0
    ordk = np.where(neg, ~u, u | 0x80000000).astype(np.uint32)
    return np.where(kept, ordk, 0).astype(np.uint32)


def _select_threshold(key, k, kept=None):
    pre, exact, top = 0, False, 31
    if kept is not None:
        # the kernel starts below the bits that every kept key shares
        kmax, kmin = int(key.max()), int(key[kept].min())
        diff = kmax ^ kmin
        top = diff.bit_length() - 1
        pre = kmax if top < 0 else kmax & ~((2 << top) - 1)
    for bit in range(top, -1, -1):
        c = pre | (1 << bit)
        cnt = int((key >= c).sum())
        if cnt >= k:
            pre = c
            if cnt == k:
                exact = True
                break
    if exact:
        return np.nonzero(key >= pre)[0]
    above = np.nonzero(key > pre)[0]
    equal = np.nonzero(key == pre)[0]          # ascending expert id
    return np.sort(np.concatenate([above, equal[:k - len(above)]]))


def _select_sort(sb, kept, k):
    e = np.nonzero(kept)[0]
    order = sorted(e.tolist(), key=lambda i: (-float(sb[i]), i))
    return np.sort(np.array(order[:k]))


def test_threshold_rule_matches_sorted_choice():
    rng = np.random.default_rng(0)
    E = 256
    for trial in range(3000):
        k = int(rng.integers(1, 9))
        mode = trial % 4
        if mode == 0:
            sb = rng.uniform(-0.05, 1.05, E)
        elif mode == 1:        # a handful of distinct values: many exact ties
            sb = rng.choice(np.array([0.25, 0.5, 0.5 + 2 ** -20, 0.75, -0.0, 0.0]), E)
        elif mode == 2:        # ties at the k-th place with some above it
            sb = np.full(E, 0.5)
            sb[rng.choice(E, int(rng.integers(0, k)), replace=False)] = 0.75
        else:                  # neighbouring floats
            sb = 0.5 + rng.integers(0, 6, E) * np.float32(2 ** -24)
        sb = sb.astype(np.float32)
        groups = rng.choice(8, int(rng.integers(4, 9)), replace=False)
        kept = np.isin(np.arange(E) // 32, groups)
        if trial % 7 == 6:     # exactly k candidates
            kept = np.zeros(E, bool)
            kept[rng.choice(E, k, replace=False)] = True
        key = _ord_keys(sb, kept)
        exp = _select_sort(sb, kept, k)
        got = _select_threshold(key, k)
        assert np.array_equal(got, exp), (trial, k, got, exp)
        got = _select_threshold(key, k, kept)
        assert np.array_equal(got, exp), (trial, k, "prefix start", got, exp)
