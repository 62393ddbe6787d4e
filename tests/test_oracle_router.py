"""Pins of the fp64 router oracle (oracle/router.py) against things other than itself:
brute-force ranking, scipy's softmax, closed forms for k = 1 and k = E, the
cancellation identity (renormalised top-k probabilities = softmax of the selected
logits), ties, and the scalar loop version."""
import itertools

import numpy as np
import pytest
from scipy.special import softmax

from oracle import router


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


@pytest.mark.parametrize("E,k", [(1, 1), (2, 1), (4, 2), (6, 3), (5, 5)])
def test_brute_force_ranking(E, k):
    g = _rng(10 + E * 7 + k)
    # few distinct values so ties are common
    lg = g.integers(-3, 3, size=(200, E)).astype(np.float64) * 0.5
    idx, prob = router.route_topk(lg, k)
    for t in range(lg.shape[0]):
        ranked = sorted(range(E), key=lambda e: (-lg[t, e], e))[:k]
        assert list(idx[t]) == ranked
        sub = lg[t, ranked]
        np.testing.assert_allclose(prob[t], softmax(sub), rtol=1e-14, atol=1e-15)
        c, p = router.route_topk_scalar(lg[t], k)
        assert c == ranked
        np.testing.assert_allclose(p, prob[t], rtol=1e-14)


def test_k_equals_E_is_the_full_softmax():
    g = _rng(3)
    lg = g.standard_normal((100, 8)) * 3
    idx, prob = router.route_topk(lg, 8)
    full = softmax(lg, axis=1)
    np.testing.assert_allclose(prob, np.take_along_axis(full, idx, axis=1), rtol=1e-13)
    assert np.all(np.diff(prob, axis=1) <= 0)


def test_k1_is_argmax_with_probability_one():
    g = _rng(4)
    lg = g.standard_normal((300, 64))
    lg[5, [3, 9]] = 10.0                       # a tie at the top: the lower id wins
    idx, prob = router.route_topk(lg, 1)
    np.testing.assert_array_equal(idx[:, 0], np.argmax(lg, axis=1))
    assert idx[5, 0] == 3
    np.testing.assert_array_equal(prob, 1.0)


def test_all_equal_logits():
    idx, prob = router.route_topk(np.zeros((3, 16)), 4)
    np.testing.assert_array_equal(idx, np.tile(np.arange(4), (3, 1)))
    np.testing.assert_allclose(prob, 0.25, rtol=0, atol=1e-15)


def test_invariants_and_large_logits():
    g = _rng(5)
    lg = g.standard_normal((500, 256)) * 30     # exp would overflow without the max shift
    for k in (1, 2, 8, 16):
        idx, prob = router.route_topk(lg, k)
        assert np.all(np.isfinite(prob))
        np.testing.assert_allclose(prob.sum(axis=1), 1.0, rtol=1e-13)
        assert np.all(np.diff(prob, axis=1) <= 1e-300)
        assert all(len(set(r)) == k for r in idx)
        # every selected logit >= every unselected one
        sel = np.take_along_axis(lg, idx, axis=1).min(axis=1)
        mask = np.ones_like(lg, dtype=bool)
        np.put_along_axis(mask, idx, False, axis=1)
        rest = np.where(mask, lg, -np.inf).max(axis=1)
        assert np.all(sel >= rest)


def test_matches_the_input_generator_router():
    """The seeded inputs route with their own code (softmax, stable top-k, renormalise)."""
    from moe_inputs.generate import route_topk as gen_route
    g = _rng(6)
    lg = g.standard_normal((400, 8)).astype(np.float32)
    i1, p1 = router.route_topk(lg, 2)
    i2, p2 = gen_route(lg, 2)
    np.testing.assert_array_equal(i1, i2)
    np.testing.assert_allclose(p1, p2, rtol=1e-6)


def test_rejects_bad_k():
    with pytest.raises(ValueError):
        router.route_topk(np.zeros((2, 4)), 5)
    with pytest.raises(ValueError):
        router.route_topk(np.zeros((2, 4)), 0)
