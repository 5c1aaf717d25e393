"""Pins of the oracle's temperature / top-k / top-p filter.

Each test checks the oracle against an independent formulation: brute-force
counting definitions on small rows, scipy's softmax, or a special case whose
answer is fixed (argmax, uniform over a tie group).
"""
import math

import numpy as np
import pytest
from scipy.special import softmax

from oracle.sampling import filter_logits


def brute_force_filter(z, T, k, top_p):
    """Counting definitions, O(V^2), no sorting or partitioning."""
    z = [float(x) for x in z]
    V = len(z)
    if 0 < k < V:
        kept = [v for v in range(V) if sum(1 for u in range(V) if z[u] > z[v]) < k]
    else:
        kept = list(range(V))
    m = max(z[v] for v in kept)
    w = {v: math.exp((z[v] - m) / T) for v in kept}
    tot = math.fsum(w.values())
    p = {v: w[v] / tot for v in kept}
    near = False
    if top_p < 1:
        new = []
        for v in kept:
            above = math.fsum(p[u] for u in kept if z[u] > z[v])
            near |= abs(above - top_p) < 1e-9
            if above < top_p or all(z[v] >= z[u] for u in kept):
                new.append(v)
        kept = new
    tot = math.fsum(w[v] for v in kept)
    return kept, [w[v] / tot for v in kept], near


def test_random_rows_match_brute_force():
    rng = np.random.default_rng(7)
    checked = 0
    for trial in range(400):
        V = int(rng.integers(1, 40))
        z = np.round(rng.normal(0, 2, V) * 2) / 2   # coarse grid -> many exact ties
        k = int(rng.integers(0, V + 3))
        top_p = float(rng.choice([0.3, 0.5, 0.8, 0.9, 0.95, 1.0]))
        T = float(rng.choice([0.5, 1.0, 2.0]))
        f = filter_logits(z, T, k, top_p)
        ids, probs, near = brute_force_filter(z, T, k, top_p)
        if near:
            continue
        assert list(f.ids) == ids, (trial, z, k, top_p)
        np.testing.assert_allclose(f.probs, probs, rtol=1e-12, atol=0)
        checked += 1
    assert checked > 300


def test_top_k_is_tie_inclusive():
    z = np.array([1.0, 5.0, 3.0, 3.0, 3.0, 0.0])
    f = filter_logits(z, 1.0, 2, 1.0)        # 2nd largest is 3.0, shared by three ids
    assert list(f.ids) == [1, 2, 3, 4]
    f = filter_logits(z, 1.0, 1, 1.0)
    assert list(f.ids) == [1] and f.probs[0] == 1.0


def test_top_k_one_with_tied_max_is_uniform_over_ties():
    z = np.array([2.0, 7.0, 7.0, -1.0])
    f = filter_logits(z, 1.0, 1, 1.0)
    assert list(f.ids) == [1, 2]
    np.testing.assert_array_equal(f.probs, [0.5, 0.5])


def test_greedy_is_lowest_id_argmax():
    z = np.array([0.0, 4.0, 9.0, 9.0, 1.0])
    for k, p in [(0, 1.0), (2, 0.5), (50, 0.95)]:
        f = filter_logits(z, 0.0, k, p)
        assert list(f.ids) == [2] and list(f.probs) == [1.0]


def test_filters_off_is_softmax():
    rng = np.random.default_rng(3)
    for T in (0.7, 1.0, 1.8):
        z = rng.normal(0, 3, 500)
        f = filter_logits(z, T, 0, 1.0)
        assert list(f.ids) == list(range(500))
        np.testing.assert_allclose(f.probs, softmax(z / T), rtol=1e-12)
        f2 = filter_logits(z, T, 500, 1.0)      # k >= V is off too
        np.testing.assert_array_equal(f2.probs, f.probs)


def test_top_k_only_is_softmax_over_the_k_largest():
    rng = np.random.default_rng(4)
    z = rng.normal(0, 3, 2000)          # continuous -> no ties
    f = filter_logits(z, 1.0, 50, 1.0)
    top = np.sort(np.argsort(z)[-50:])
    assert list(f.ids) == list(top)
    np.testing.assert_allclose(f.probs, softmax(z[top]), rtol=1e-12)


def test_top_p_to_zero_keeps_the_top_group_only():
    z = np.array([0.5, 3.0, 2.9, 3.0, 1.0])
    f = filter_logits(z, 1.0, 0, 1e-12)
    assert list(f.ids) == [1, 3]
    z2 = np.array([0.5, 3.0, 2.9, 1.0])
    f2 = filter_logits(z2, 1.0, 3, 1e-12)
    assert list(f2.ids) == [1] and f2.probs[0] == 1.0


def test_top_p_cut_hand_computed():
    # probabilities 0.5, 0.3, 0.2 (logits are their logs): top_p 0.6 keeps the
    # tokens whose mass-above is 0 and 0.5 (< 0.6), drops the one with 0.8.
    z = np.log(np.array([0.3, 0.5, 0.2]))
    f = filter_logits(z, 1.0, 0, 0.6)
    assert list(f.ids) == [0, 1]
    np.testing.assert_allclose(f.probs, [0.375, 0.625], rtol=1e-12)
    f = filter_logits(z, 1.0, 0, 0.5)       # mass above 0.3-token is 0.5: not < 0.5
    assert list(f.ids) == [1]
    f = filter_logits(z, 1.0, 0, 0.81)
    assert list(f.ids) == [0, 1, 2]


def test_output_is_a_distribution_with_ascending_ids():
    rng = np.random.default_rng(5)
    for _ in range(50):
        z = rng.normal(0, 3, 300).astype(np.float32).astype(np.float64)
        f = filter_logits(z, 1.0, 50, 0.95)
        assert np.all(np.diff(f.ids) > 0)
        assert np.all(f.probs > 0)
        assert abs(math.fsum(f.probs) - 1.0) < 1e-12
        assert 1 <= len(f.ids) <= 50


@pytest.mark.parametrize("V", [1, 2])
def test_tiny_vocabularies(V):
    z = np.arange(V, dtype=np.float64)
    f = filter_logits(z, 1.0, 50, 0.95)
    assert f.ids[-1] == V - 1 and abs(f.probs.sum() - 1) < 1e-15
