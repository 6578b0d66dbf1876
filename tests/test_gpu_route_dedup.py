"""GPU parity: routing and distinct-expert dedup against the oracle."""
import numpy as np
import pytest
import torch

import workloads as W
from helpers import flush
from oracle import dedup_sorted, route_topk_softmax

pytestmark = pytest.mark.gpu


def _route_gpu(lg, k):
    import slot_cache_routed_amd._lib as L
    T, E = lg.shape
    d = torch.from_numpy(np.ascontiguousarray(lg)).cuda()
    ids = torch.full((max(T, 1), k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((max(T, 1), k), -7.0, dtype=torch.float32, device="cuda")
    L.route(d, T, E, k, ids, w, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return ids.cpu().numpy()[:T], w.cpu().numpy()[:T]


def _cases():
    return [
        ("tiny", W.logits_normal(1, 0, 32, 8), 2),
        ("short_prefill_96", W.logits_with_chosen(2, 96, 512, 10, 160)[0], 10),
        ("layer_view_600", W.logits_normal(3, 0, 600, 8), 2),
        ("decode_step", W.zipf_gumbel_logits(4, 0, 0, 4, 512), 10),
        ("long_prefill_4096", W.logits_normal(5, 0, 4096, 512), 10),
        ("max_experts_k32", W.logits_normal(6, 0, 33, 4096), 32),
        ("one_expert", W.logits_normal(7, 0, 5, 1), 1),
        ("ragged_E_100", W.logits_normal(8, 0, 77, 100), 7),
    ]


@pytest.mark.parametrize("name,lg,k", _cases(), ids=[c[0] for c in _cases()])
def test_route_matches_oracle(name, lg, k):
    flush(f"route {name} {lg.shape} k={k}")
    ids, w = _route_gpu(lg, k)
    rid, rw = route_topk_softmax(lg, k)
    assert np.array_equal(ids, rid), "expert ids are bit-exact"
    diff = np.abs(w.view(np.int32).astype(np.int64) - rw.view(np.int32).astype(np.int64))
    # fp64 exp on either side agrees to well under one fp32 ulp; a value can
    # only differ when the fp64 result sits on an fp32 rounding boundary
    assert diff.max() <= 1
    assert np.count_nonzero(diff) <= max(1, diff.size // 100000)


def test_route_ties_and_empty():
    lg = np.array([[1.0, 3.0, 3.0, 0.5, 3.0, -2.0]] * 3, dtype=np.float32)
    ids, w = _route_gpu(lg, 4)
    assert ids[0].tolist() == [1, 2, 4, 0]
    ids, w = _route_gpu(np.zeros((0, 8), np.float32), 2)
    assert ids.shape == (0, 2)


def _dedup_gpu(ids, E):
    import slot_cache_routed_amd._lib as L
    n = ids.size
    d = torch.from_numpy(np.ascontiguousarray(ids.astype(np.int32))).cuda()
    lmax = min(n, E)
    dist = torch.full((max(lmax, 1),), -9, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    inv = torch.full((max(n, 1),), -9, dtype=torch.int32, device="cuda")
    L.dedup(d, n, E, dist, cnt, inv, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return dist.cpu().numpy()[:lmax], int(cnt.item()), inv.cpu().numpy()[:n]


@pytest.mark.parametrize("n,E", [(64, 8), (960, 512), (40, 512), (40960, 512), (1200, 8), (3000, 4096),
                                 (7, 8192), (1, 1)])
def test_dedup_matches_oracle(n, E):
    flush(f"dedup n={n} E={E}")
    ids = W.uniform_ids(9, n, E)
    got = _dedup_gpu(ids, E)
    ref = dedup_sorted(ids, E)
    assert np.array_equal(got[0], ref[0]) and got[1] == ref[1] and np.array_equal(got[2], ref[2])


def test_dedup_short_prefill_has_160_and_ignores_invalid():
    lg, D = W.logits_with_chosen(2, 96, 512, 10, 160)
    rid, _ = route_topk_softmax(lg, 10)
    dist, cnt, inv = _dedup_gpu(rid.reshape(-1), 512)
    assert cnt == 160 and dist[:160].tolist() == D.tolist() and np.all(dist[160:] == 512)
    ids = np.array([3, -1, 9, 3, 12, 0], np.int32)
    dist, cnt, inv = _dedup_gpu(ids, 10)
    assert cnt == 3 and dist.tolist() == [0, 3, 9, 10, 10, 10] and inv.tolist() == [1, -1, 2, 1, -1, 0]


def test_route_signed_zeros_tie_and_minus_infinity():
    # -0.0 and +0.0 are equal logits (ties go to the lower id); -inf logits are
    # never chosen while finite ones remain
    lg = np.array([[0.0, -0.0, -np.inf, 0.0, -1.0, -np.inf, -0.0, 2.0]] * 4, dtype=np.float32)
    lg[1] = lg[1][::-1]
    ids, w = _route_gpu(lg, 5)
    rid, rw = route_topk_softmax(lg, 5)
    assert np.array_equal(ids, rid)
    assert ids[0].tolist() == [7, 0, 1, 3, 6]
    assert np.array_equal(w.view(np.int32), rw.view(np.int32))


@pytest.mark.parametrize("E,k", [(512, 10), (4096, 32), (100, 7)])
def test_route_with_many_equal_logits(E, k):
    # logits from three values: equal keys within one lane's slots and across
    # lanes in every round; rows of one value throughout choose ids 0..k-1
    g = np.random.default_rng(E + k)
    lg = g.integers(0, 3, size=(64, E)).astype(np.float32)
    lg[5] = 1.0
    lg[9] = -2.5
    lg[11, : E // 2] = 0.0
    lg[11, E // 2:] = 0.0 * -1.0
    ids, w = _route_gpu(lg, k)
    rid, rw = route_topk_softmax(lg, k)
    assert np.array_equal(ids, rid)
    assert ids[5].tolist() == list(range(k)) and ids[9].tolist() == list(range(k))
    diff = np.abs(w.view(np.int32).astype(np.int64) - rw.view(np.int32).astype(np.int64))
    assert diff.max() <= 1
