"""Pins of the router top-k oracle (oracle/router.py) against facts that
do not come from the oracle's own ranking loop: the order statistics of the
scores, the renormalised full softmax, and closed forms of the weights."""
import math

import numpy as np
import pytest

from oracle import router


def _scores(seed, T, E, ties=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, E)).astype(np.float32)
    if ties:                                   # few distinct values: many exact ties
        x = np.round(x * 2).astype(np.float32) / np.float32(2)
    return x


@pytest.mark.parametrize("ties", [False, True])
@pytest.mark.parametrize("E,K", [(8, 2), (64, 6), (256, 8)])
def test_ids_are_the_k_largest_ties_to_lower_id(E, K, ties):
    x = _scores(1, 40, E, ties)
    ids, _ = router.router_topk(x, K)
    for t in range(x.shape[0]):
        # independent ranking: lexsort by (score desc, id asc)
        ref = np.lexsort((np.arange(E), -x[t].astype(np.float64)))[:K]
        assert list(ids[t]) == list(ref)
        sel, rest = x[t, ids[t]], np.delete(x[t], ids[t])
        assert np.all(np.diff(sel.astype(np.float64)) <= 0)          # descending
        if rest.size:
            assert sel.min() >= rest.max()                            # nothing larger left out


def test_weights_equal_renormalised_full_softmax():
    x = _scores(2, 30, 64)
    ids, w = router.router_topk(x, 6)
    for t in range(30):
        v = x[t].astype(np.float64)
        p = np.exp(v - v.max()); p /= p.sum()                         # softmax over all experts
        top = np.argsort(-p, kind="stable")[:6]
        assert list(top) == list(ids[t])
        ref = p[top] / p[top].sum()                                   # renormalised over the top-6
        np.testing.assert_allclose(w[t], ref, rtol=2e-7, atol=0)


def test_weight_closed_forms():
    x = np.array([[0.0, math.log(3.0), -50.0, -51.0]], np.float32)
    ids, w = router.router_topk(x, 2)
    assert list(ids[0]) == [1, 0]
    np.testing.assert_allclose(w[0], [0.75, 0.25], rtol=1e-6)         # e^ln3 : e^0 = 3 : 1
    ids1, w1 = router.router_topk(x, 1)
    assert list(ids1[0]) == [1] and w1[0, 0] == 1.0
    ids4, w4 = router.router_topk(np.zeros((1, 4), np.float32), 4)   # all equal
    assert list(ids4[0]) == [0, 1, 2, 3] and np.all(w4 == 0.25)


def test_bias_selection_and_weights():
    x = np.array([[1.0, 0.9, 0.8, 0.0]], np.float32)
    b = np.array([0.0, 0.0, 0.5, 0.0], np.float32)
    ids, w = router.router_topk(x, 2, bias=b)                         # scores 1.0 0.9 1.3 0.0
    assert list(ids[0]) == [2, 0]
    np.testing.assert_allclose(w[0], [1 / (1 + math.exp(-0.3)), 1 / (1 + math.exp(0.3))], rtol=1e-6)
    ids2, w2 = router.router_topk(x, 2, bias=b, bias_in_weights=False)
    assert list(ids2[0]) == [2, 0]                                    # same selection
    np.testing.assert_allclose(w2[0], [1 / (1 + math.exp(0.2)), 1 / (1 + math.exp(-0.2))], rtol=1e-6)
    z = np.zeros(4, np.float32)
    assert np.array_equal(router.router_topk(x, 3, bias=z)[0], router.router_topk(x, 3)[0])


def test_fp32_bias_add_decides_ties():
    # 1 + 2^-24 rounds to 1 in fp32: the biased scores tie and the lower id wins,
    # whereas a float64 add would have ranked expert 1 first
    x = np.array([[1.0, 1.0]], np.float32)
    b = np.array([0.0, 2.0 ** -24], np.float32)
    ids, _ = router.router_topk(x, 1, bias=b)
    assert ids[0, 0] == 0


def test_nan_ranks_last():
    x = np.array([[np.nan, -1e30, 0.5]], np.float32)
    ids, w = router.router_topk(x, 2)
    assert list(ids[0]) == [2, 1]
    # below -inf too, whatever its id
    x = np.array([[np.nan, -np.inf, np.inf, -0.0, 0.0]], np.float32)
    ids, _ = router.router_topk(x, 5)
    assert list(ids[0]) == [2, 3, 4, 1, 0]                             # -0 and +0 tie: lower id first
