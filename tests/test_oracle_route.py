"""Pins of the router top-k: selection by repeated arg-max on tiny inputs
with constructed ties, k = E, and softmax weights against scipy (CPU only)."""
import numpy as np
import pytest
from scipy.special import softmax

from oracle.route import route_topk


def brute_topk(row, k):
    """Repeated scan: pick the largest remaining logit, the lowest index on
    equal values."""
    left = list(range(len(row)))
    out = []
    for _ in range(k):
        best = left[0]
        for e in left[1:]:
            if row[e] > row[best]:
                best = e
        out.append(best)
        left.remove(best)
    return out


@pytest.mark.parametrize("seed", range(5))
def test_selection_with_ties(seed):
    rng = np.random.default_rng(seed)
    T, E = 64, 7
    # few distinct values -> many ties
    lg = rng.integers(-2, 3, size=(T, E)).astype(np.float32) * np.float32(0.5)
    for k in range(1, E + 1):
        ids, w = route_topk(lg, k)
        for t in range(T):
            assert ids[t].tolist() == brute_topk(lg[t].tolist(), k)
        assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-15)


def test_k_equals_E_returns_all():
    lg = np.array([[0.1, 3.0, -1.0, 3.0]], np.float32)
    ids, w = route_topk(lg, 4)
    assert ids.tolist() == [[1, 3, 0, 2]]
    assert w[0, 0] == w[0, 1]


def test_weights_are_softmax_of_selected():
    rng = np.random.default_rng(9)
    lg = rng.normal(size=(100, 32)).astype(np.float32) * np.float32(3)
    ids, w = route_topk(lg, 8)
    sel = np.take_along_axis(lg.astype(np.float64), ids, 1)
    assert np.allclose(w, softmax(sel, axis=1), rtol=1e-14, atol=0)
    assert (np.diff(w, axis=1) <= 0).all()


def test_exact_fp32_selection_near_ties():
    """Logits that differ in the last fp32 bit are ordered by value."""
    a = np.float32(1.0)
    b = np.nextafter(a, np.float32(2))
    lg = np.array([[a, b, a, b]], np.float32)
    ids, _ = route_topk(lg, 3)
    assert ids.tolist() == [[1, 3, 0]]
