"""Pins for the LRU slot-bank oracle (CPU)."""
from collections import OrderedDict

import numpy as np
import pytest

import workloads as W
from conftest import read_golden
from oracle import SlotBankState, dedup_sorted, ensure_slots, route_topk_softmax
from oracle.lru import ERR_CAPACITY, STAT_EVICTIONS, STAT_HITS, STAT_MISSES, STAT_QUERIES


def _bijection(st):
    for s in range(st.S):
        key = int(st.slot_key[s])
        if key >= 0:
            assert st.key_to_slot[key] == s
    res = np.nonzero(st.key_to_slot >= 0)[0]
    for key in res:
        assert st.slot_key[st.key_to_slot[key]] == key


def _run_queries(st, layer, distinct, width, record):
    splits = []
    for q0 in range(0, distinct.size, width):
        ms, mk = ensure_slots(st, layer, distinct[q0:q0 + width], record)
        splits.append(len(ms))
    return splits


def test_short_prefill_admits_128_then_32_and_records_no_stats():
    row = [r for r in read_golden("lru_query_splits.txt") if r[0] == "short_prefill_96"][0]
    n_distinct, width, S = int(row[1]), int(row[2]), int(row[3])
    want = [int(v) for v in row[4:]]
    cfg = W.C2
    lg, D = W.logits_with_chosen(cfg.seed, cfg.T, cfg.shape.E, cfg.shape.k, n_distinct)
    ids, _ = route_topk_softmax(lg, cfg.shape.k)
    distinct, cnt, _ = dedup_sorted(ids.reshape(-1), cfg.shape.E)
    assert cnt == n_distinct
    fill = W.bank_prefilled(cfg.seed, S, cfg.L, cfg.shape.E, 600, exclude_layer=0)
    st = SlotBankState.from_fill(fill)
    before_keys = st.slot_key.copy()
    splits = _run_queries(st, 0, distinct, width, record=False)
    assert splits == want
    assert np.all(st.stats == 0) and np.all(st.decode_freq == 0)
    assert st.clock == 600 + len(want)
    # all 160 experts resident; the 500 empty slots absorb them, lowest index first
    slots = st.key_to_slot[D]
    assert np.all(slots >= 0)
    empty = np.nonzero(before_keys < 0)[0]
    assert sorted(slots.tolist()) == empty[:n_distinct].tolist()
    # the other layers' 600 experts stay resident
    assert np.array_equal(st.slot_key[before_keys >= 0], before_keys[before_keys >= 0])
    _bijection(st)


def test_one_layer_cache_filled_three_per_query():
    row = [r for r in read_golden("lru_query_splits.txt") if r[0] == "layer_view_s8"][0]
    n, width, S = int(row[1]), int(row[2]), int(row[3])
    want = [int(v) for v in row[4:]]
    fill = W.bank_prefilled(3, S, 48, 8, S, exclude_layer=0)      # full of other layers' experts
    st = SlotBankState.from_fill(fill)
    distinct = np.arange(n, dtype=np.int32)
    assert _run_queries(st, 0, distinct, width, record=False) == want
    assert np.all(st.key_to_slot[:8] >= 0)
    assert np.all(st.stats == 0)
    _bijection(st)


def test_earlier_queries_are_evicted_last():
    # a full bank of old keys; query 2's misses must take older slots, never query 1's
    S, E, L = 12, 64, 2
    sk = np.arange(S, dtype=np.int32) + E          # layer-1 keys
    stamps = np.arange(1, S + 1, dtype=np.uint64)
    st = SlotBankState(S, L, E, sk, stamps)
    st.clock = S
    q1 = np.array([0, 1, 2, 3], np.int32)
    q2 = np.array([4, 5, 6, 7], np.int32)
    s1, _ = ensure_slots(st, 0, q1, False)
    s2, _ = ensure_slots(st, 0, q2, False)
    assert not set(s1) & set(s2)
    assert s1 == [0, 1, 2, 3] and s2 == [4, 5, 6, 7]     # oldest stamps first
    assert np.all(st.key_to_slot[:8] >= 0)


def test_hits_are_touched_and_never_evicted_by_their_own_query():
    S, E = 4, 16
    st = SlotBankState(S, 1, E)
    ensure_slots(st, 0, [0, 1, 2, 3], True)              # fills all four
    ensure_slots(st, 0, [4], True)                       # evicts expert 0 (slot 0)
    assert st.key_to_slot[0] == -1 and st.key_to_slot[4] == 0
    ms, mk = ensure_slots(st, 0, [1, 5], True)           # 1 hits; 5 must not evict 1
    assert mk == [5] and st.key_to_slot[1] >= 0 and ms == [2]
    assert st.stats[STAT_HITS] == 1 and st.stats[STAT_MISSES] == 6
    assert st.stats[STAT_EVICTIONS] == 2 and st.stats[STAT_QUERIES] == 3
    assert st.decode_freq[1] == 2 and st.decode_freq[5] == 1


def test_matches_a_textbook_recency_list_lru_when_stamps_are_distinct():
    # one expert per query makes every stamp distinct, so the policy is classic LRU
    g = np.random.default_rng(11)
    S, E = 16, 64
    st = SlotBankState(S, 1, E)
    book = OrderedDict()
    for step in range(3000):
        e = int(min(g.zipf(1.3), E) - 1)
        evicted_book = None
        if e in book:
            book.move_to_end(e)
        else:
            if len(book) == S:
                evicted_book, _ = book.popitem(last=False)
            book[e] = True
        before = set(np.nonzero(st.key_to_slot >= 0)[0].tolist())
        ensure_slots(st, 0, [e], True)
        after = set(np.nonzero(st.key_to_slot >= 0)[0].tolist())
        assert after == set(book.keys()), step
        gone = before - after
        assert gone == ({evicted_book} if evicted_book is not None else set())
    _bijection(st)


def test_capacity_violation_sets_the_error_bit():
    st = SlotBankState(4, 1, 16)
    ms, mk = ensure_slots(st, 0, [0, 1, 2, 3, 4], False)
    assert len(ms) == 4 and st.err & ERR_CAPACITY
    assert st.key_to_slot[4] == -1


def test_sentinel_only_query_ticks_the_clock_and_admits_nothing():
    st = SlotBankState(4, 1, 16)
    ms, _ = ensure_slots(st, 0, [16, 16, 16], True)
    assert ms == [] and st.clock == 1 and st.stats[STAT_QUERIES] == 1
