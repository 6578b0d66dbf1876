"""Pins for the distinct-expert oracle (CPU)."""
import numpy as np

import workloads as W
from oracle import dedup_sorted, route_topk_softmax


def test_matches_python_set_and_inverse_maps_back():
    g = np.random.default_rng(5)
    for n, E in [(64, 8), (960, 512), (40, 512), (3000, 100)]:
        ids = g.integers(0, E, size=n).astype(np.int32)
        distinct, cnt, inv = dedup_sorted(ids, E)
        ref = sorted(set(ids.tolist()))
        assert cnt == len(ref)
        assert distinct.size == min(n, E)
        assert distinct[:cnt].tolist() == ref
        assert np.all(distinct[cnt:] == E)
        assert np.array_equal(distinct[inv], ids)


def test_invalid_ids_are_not_experts():
    distinct, cnt, inv = dedup_sorted(np.array([3, -1, 9, 3, 12, 0], np.int32), 10)
    assert cnt == 3 and distinct.tolist() == [0, 3, 9, 10, 10, 10]
    assert inv.tolist() == [1, -1, 2, 1, -1, 0]


def test_short_prefill_chunk_routes_to_160_experts():
    # FreeToken PR #676, Tests: a 96-token chunk routing to 160 experts
    lg, _ = W.logits_with_chosen(2, 96, 512, 10, 160)
    ids, _ = route_topk_softmax(lg, 10)
    distinct, cnt, _ = dedup_sorted(ids.reshape(-1), 512)
    assert cnt == 160 and distinct.size == 512
