"""Pins for the align oracle (CPU)."""
import numpy as np
import pytest

import workloads as W
from conftest import read_golden
from oracle import align_blocks, align_capacity


def _check_invariants(ids, bucket_of, Nb, B, out):
    n = ids.size
    sr, bb = out["sorted_routes"], out["block_bucket"]
    P = out["n_post_pad"]
    assert P % B == 0 and sr.size == out["capacity"] == align_capacity(n, Nb, B)
    valid = [r for r in range(n) if 0 <= bucket_of[r] < Nb]
    seen = {}
    for pos in range(P):
        r = int(sr[pos])
        if r == n:
            continue
        assert r not in seen, "a route lands once"
        seen[r] = pos
        assert bb[pos // B] == bucket_of[r], "in a block of its own bucket"
    assert sorted(seen) == valid
    assert np.all(sr[P:] == n) and np.all(bb[P // B:] == -1)
    # per-bucket padding and active list
    counts = np.bincount(np.asarray([bucket_of[r] for r in valid], np.int64), minlength=Nb)
    act = np.nonzero(counts)[0]
    assert out["active_buckets"].tolist() == act.tolist()
    padded = -(-counts[act] // B) * B
    assert P == int(padded.sum())
    assert out["active_block_begin"].tolist() == (np.concatenate([[0], np.cumsum(padded)]) // B).tolist()


@pytest.mark.parametrize("Nb", [int(r[0]) for r in read_golden("align_bucket_counts.txt")])
@pytest.mark.parametrize("n", [40, 960, 4000])
@pytest.mark.parametrize("B", [16, 64])
def test_every_route_lands_once_in_a_block_of_its_bucket(Nb, n, B):
    ids = W.uniform_ids(4, n, Nb)
    out = align_blocks(ids, None, Nb, B)
    _check_invariants(ids, ids.tolist(), Nb, B, out)


def test_stable_argsort_closed_form():
    ids = W.uniform_ids(8, 5000, 300)
    out = align_blocks(ids, None, 300, 16)
    body = [r for r in out["sorted_routes"][:out["n_post_pad"]].tolist() if r != ids.size]
    assert body == np.argsort(ids, kind="stable").tolist()


def test_worked_example():
    g = {r[0]: [int(v) for v in r[1:]] for r in read_golden("align_worked_example.txt")}
    out = align_blocks(np.array(g["ids"], np.int32), None, g["num_buckets"][0], g["block"][0])
    assert out["sorted_routes"][:out["n_post_pad"]].tolist() == g["sorted"]
    assert out["block_bucket"][:len(g["block_bucket"])].tolist() == g["block_bucket"]
    assert out["n_post_pad"] == g["n_post_pad"][0]
    assert out["active_buckets"].tolist() == g["active"]
    assert out["active_block_begin"].tolist() == g["active_begin"]


def test_map_to_slots_drops_unmapped_and_out_of_range():
    # experts 0..7 of a layer mapped into a 1100-slot bank; expert 5 unmapped
    m = np.array([900, 13, 1024, 2, 1099, -1, 400, 77], np.int32)
    ids = W.uniform_ids(3, 1200, 8)
    ids[7] = 9       # not an expert of the layer
    out = align_blocks(ids, m, 1100, 16)
    bucket_of = [int(m[i]) if 0 <= i < 8 else -1 for i in ids.tolist()]
    _check_invariants(ids, bucket_of, 1100, 16, out)
    assert 5 not in [ids[r] for r in out["sorted_routes"] if r < ids.size]


def test_bucket_order_makes_slot_and_expert_layouts_agree_when_the_map_is_monotone():
    ids = W.uniform_ids(6, 300, 8)
    m = np.array([3, 10, 11, 40, 41, 42, 90, 91], np.int32)
    a = align_blocks(ids, None, 8, 16)
    b = align_blocks(ids, m, 128, 16)
    assert a["n_post_pad"] == b["n_post_pad"]
    assert a["sorted_routes"][:a["n_post_pad"]].tolist() == b["sorted_routes"][:b["n_post_pad"]].tolist()
    assert (m[a["active_buckets"]]).tolist() == b["active_buckets"].tolist()
