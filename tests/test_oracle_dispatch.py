"""Pins of the oracle's counting sort (dispatch) and combine."""
import numpy as np
import pytest

from oracle import counting_sort, combine, permute_rows


def _dispatch_bruteforce(idx, E, n_shared):
    T, k = idx.shape
    counts = [0] * (E + n_shared)
    for t in range(T):
        for j in range(k):
            counts[idx[t, j]] += 1
    for s in range(n_shared):
        counts[E + s] = T
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    fill = list(offsets[:-1])
    dest = [[None] * k for _ in range(T)]
    src = [None] * offsets[-1]
    for t in range(T):                      # token-ascending within each expert
        for j in range(k):
            e = idx[t, j]
            dest[t][j] = fill[e]
            src[fill[e]] = t
            fill[e] += 1
    for s in range(n_shared):
        for t in range(T):
            src[offsets[E + s] + t] = t
    return counts, offsets, dest, src


def _random_routing(rng, T, E, k, skew=False):
    if skew:
        p = 1.0 / np.arange(1, E + 1) ** 1.5
        p /= p.sum()
        return np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    return np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("T,E,k,ns,skew", [(1, 1, 1, 0, False), (37, 8, 2, 0, False),
                                          (64, 16, 4, 1, True), (100, 33, 7, 0, True),
                                          (5, 64, 8, 1, False)])
def test_counting_sort_matches_bruteforce(T, E, k, ns, skew):
    rng = np.random.default_rng(T * 7 + E)
    idx = _random_routing(rng, T, E, k, skew)
    counts, offsets, dest, src = counting_sort(idx, E, ns)
    bc, bo, bd, bs = _dispatch_bruteforce(idx, E, ns)
    assert counts.tolist() == bc and offsets.tolist() == bo
    assert dest.tolist() == bd and src.tolist() == bs


def test_counting_sort_invariants():
    rng = np.random.default_rng(5)
    T, E, k = 300, 50, 6
    idx = _random_routing(rng, T, E, k, skew=True)
    counts, offsets, dest, src = counting_sort(idx, E, 0)
    assert counts.sum() == T * k
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(np.sort(dest.ravel()), np.arange(T * k))      # bijection
    for t in range(T):
        for j in range(k):
            assert src[dest[t, j]] == t
            assert offsets[idx[t, j]] <= dest[t, j] < offsets[idx[t, j] + 1]
    for e in range(E):                                                   # token-ascending
        assert np.all(np.diff(src[offsets[e]:offsets[e + 1]]) > 0)


def test_one_hot_combine_is_inverse_permutation():
    rng = np.random.default_rng(6)
    T, E, H = 40, 7, 16
    idx = rng.integers(0, E, (T, 1)).astype(np.int32)
    counts, offsets, dest, src = counting_sort(idx, E, 0)
    x = rng.standard_normal((T, H)).astype(np.float32)
    y_perm = permute_rows(x, src)
    w = np.ones((T, 1), np.float32)          # k = 1 renormalises to exactly 1
    assert np.array_equal(combine(y_perm, dest, w), x)


def test_combine_order_and_shared():
    T, H, k = 3, 2, 2
    y = np.arange((T * k + T) * H, dtype=np.float32).reshape(T * k + T, H)
    dest = np.array([[1, 0], [2, 5], [4, 3]], np.int32)
    w = np.array([[0.75, 0.25], [0.5, 0.5], [1.0, 0.0]], np.float32)
    out = combine(y, dest, w, n_shared=1)
    ref = np.stack([w[t, 0] * y[dest[t, 0]] + w[t, 1] * y[dest[t, 1]] + y[T * k + t] for t in range(T)])
    assert np.array_equal(out, ref)
