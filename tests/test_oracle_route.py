"""Pins of the oracle's router: logits, top-k with ties, renormalised softmax."""
import numpy as np
import pytest

from oracle import router_logits, topk_softmax


def _topk_bruteforce(logits, k):
    """sorted() with the key (-value, index): largest first, lower index wins ties."""
    T, E = logits.shape
    idx = np.array([sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k] for t in range(T)])
    return idx


@pytest.mark.parametrize("seed", range(5))
def test_topk_matches_bruteforce_with_heavy_ties(seed):
    rng = np.random.default_rng(seed)
    T, E = 50, 33
    # few distinct values -> many ties; include +-0
    vals = np.array([-1.5, -0.0, 0.0, 0.25, 1.0, 2.0], np.float32)
    logits = vals[rng.integers(0, len(vals), (T, E))]
    for k in (1, 2, 5, 8, E):
        idx, w = topk_softmax(logits, k)
        assert np.array_equal(idx, _topk_bruteforce(logits, k))


def test_plus_minus_zero_tie_and_ulp_neighbours():
    one = np.float32(1.0)
    up = np.nextafter(one, np.float32(2))
    logits = np.array([[-0.0, 0.0, -0.0, 0.0],
                       [0.0, -0.0, 0.0, -0.0],
                       [one, up, one, up],
                       [up, one, up, one]], np.float32)
    idx, _ = topk_softmax(logits, 2)
    assert idx.tolist() == [[0, 1], [0, 1], [1, 3], [0, 2]]


def test_zero_router_weight_ties_everything():
    rng = np.random.default_rng(0)
    T, H, E, k = 17, 64, 12, 5
    x = rng.standard_normal((T, H)).astype(np.float32)
    l = router_logits(x, np.zeros((E, H), np.float32))
    idx, w = topk_softmax(l, k)
    assert np.all(idx == np.arange(k)[None, :])
    assert np.all(w == np.float32(1.0) / np.float32(k))


def test_router_logits_exact_on_integer_inputs():
    """Small integers make every fp32 product and partial sum exact."""
    rng = np.random.default_rng(1)
    T, H, E = 7, 40, 9                       # H != E: a transposed operand would not even fit
    x = rng.integers(-4, 5, (T, H)).astype(np.float32)
    W = rng.integers(-3, 4, (E, H)).astype(np.float32)
    b = rng.integers(-2, 3, (E,)).astype(np.float32)
    l = router_logits(x, W, b)
    ref = [[sum(int(x[t, h]) * int(W[e, h]) for h in range(H)) + int(b[e]) for e in range(E)]
           for t in range(T)]
    assert np.array_equal(l, np.array(ref, np.float32))


@pytest.mark.parametrize("seed", range(3))
def test_weights_vs_float64_full_softmax(seed):
    """Renormalised weights equal a float64 softmax over all experts restricted to
    the selected ones (within 1e-6, the Ironwood page's numeric verification, section 6)."""
    rng = np.random.default_rng(seed)
    T, E, k = 64, 128, 8
    logits = (rng.standard_normal((T, E)) * 3).astype(np.float32)
    idx, w = topk_softmax(logits, k)
    l64 = logits.astype(np.float64)
    p = np.exp(l64 - l64.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    sel = np.take_along_axis(p, idx.astype(np.int64), 1)
    ref = sel / sel.sum(1, keepdims=True)
    assert np.max(np.abs(w - ref)) <= 1e-6
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= k * 2.0 ** -23)
    # slots are ordered best first
    assert np.all(np.diff(np.take_along_axis(logits, idx.astype(np.int64), 1), axis=1) <= 0)
    assert np.all(np.diff(w, axis=1) <= 0)


def test_non_finite_logits_rejected():
    with pytest.raises(AssertionError):
        topk_softmax(np.array([[0.0, np.nan]], np.float32), 1)
