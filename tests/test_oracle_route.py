"""Pins for the routing oracle (CPU)."""
import itertools

import numpy as np
import pytest
import scipy.special

import workloads as W
from oracle import route_topk_softmax


def _ulp_diff(a, b):
    a = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(a - b)


@pytest.mark.parametrize("E,k", [(8, 2), (6, 3), (7, 1), (5, 5)])
def test_topk_set_is_the_max_sum_subset_brute_force(E, k):
    lg = W.logits_normal(101, 0, 40, E)
    ids, _ = route_topk_softmax(lg, k)
    for t in range(lg.shape[0]):
        best = max(itertools.combinations(range(E), k), key=lambda c: sum(float(lg[t, e]) for e in c))
        assert sorted(ids[t].tolist()) == sorted(best)
        vals = lg[t, ids[t]]
        assert np.all(vals[:-1] >= vals[1:]), "rank order is by descending logit"


def test_weights_equal_scipy_softmax_of_selected_logits():
    lg = W.logits_normal(1, 0, 32, 8)              # tiny workload's router logits
    for k in (2, 4, 8):
        ids, w = route_topk_softmax(lg, k)
        for t in range(lg.shape[0]):
            ref = scipy.special.softmax(lg[t, ids[t]].astype(np.float64))
            assert _ulp_diff(w[t], ref.astype(np.float32)).max() <= 1


def test_k1_weight_is_exactly_one():
    lg = W.logits_normal(7, 0, 50, 16)
    ids, w = route_topk_softmax(lg, 1)
    assert np.all(w == np.float32(1.0))
    assert np.array_equal(ids[:, 0], np.argmax(lg, axis=1))


def test_k2_closed_form_is_logistic_of_the_gap():
    lg = W.logits_normal(9, 0, 64, 8)
    ids, w = route_topk_softmax(lg, 2)
    gap = lg[np.arange(64), ids[:, 0]].astype(np.float64) - lg[np.arange(64), ids[:, 1]].astype(np.float64)
    assert _ulp_diff(w[:, 0], scipy.special.expit(gap).astype(np.float32)).max() <= 1
    assert _ulp_diff(w[:, 1], scipy.special.expit(-gap).astype(np.float32)).max() <= 1


def test_ties_go_to_the_lower_expert_id():
    lg = np.array([[1.0, 3.0, 3.0, 0.5, 3.0, -2.0]], dtype=np.float32)
    ids, w = route_topk_softmax(lg, 4)
    assert ids[0].tolist() == [1, 2, 4, 0]
    assert w[0, 0] == w[0, 1] == w[0, 2]


def test_weights_sum_to_one_and_descend_on_the_short_prefill_logits():
    lg, D = W.logits_with_chosen(2, 96, 512, 10, 160)
    ids, w = route_topk_softmax(lg, 10)
    s = w.astype(np.float64).sum(axis=1)
    assert np.all(np.abs(s - 1.0) <= 10 * 2.0 ** -24)
    assert np.all(w[:, :-1] >= w[:, 1:])
    # every token's ten chosen experts carry the +10 offset, so they are its top-10
    assert set(np.unique(ids).tolist()) == set(D.tolist())
