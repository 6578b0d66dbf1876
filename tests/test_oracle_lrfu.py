"""Pins for the LRFU (scored) eviction of the slot-bank oracle (CPU)."""
from fractions import Fraction

import numpy as np

from conftest import read_golden
from oracle import SlotBankState, ensure_slots
from oracle.lru import CRF_ONE, POLICY_LRFU, POLICY_LRU, crf_decay, pow_q32

HALF = 3037000499            # floor(2^32 * 2^-0.5): lambda = 1/2
LAMBDA1 = 1 << 31            # lambda = 1
NEAR_ONE = (1 << 32) - 1     # lambda ~ 2^-32 / ln 2: almost no decay (LFU limit)


def _bank(S, E, policy, D, L=1):
    st = SlotBankState(S, L, E)
    st.policy, st.decay_q32 = policy, D
    return st


def test_fixed_point_power_is_a_truncation_of_the_exact_power():
    # truncation only lowers the value; a squaring doubles the relative error
    # it inherits, so the loss stays within about 2n + 2 bitlen(n) Q0.32 units
    g = np.random.default_rng(0)
    for _ in range(300):
        D = int(g.integers(1, 1 << 32))
        n = int(g.integers(0, 600))
        exact = Fraction(D, 1 << 32) ** n * (1 << 32)
        p = pow_q32(D, n)
        assert p <= exact and exact - p <= 2 * n + 2 * n.bit_length() + 2
    assert pow_q32(HALF, 0) == 1 << 32 and pow_q32(LAMBDA1, 5) == 1 << 27
    assert crf_decay(CRF_ONE, 3, LAMBDA1) == CRF_ONE >> 3


def test_worked_example_where_lrfu_and_lru_disagree():
    for policy, seq, victim, evicted in read_golden("lrfu_worked_example.txt"):
        st = _bank(2, 4, POLICY_LRFU if policy == "lrfu" else POLICY_LRU, HALF)
        experts = [int(e) for e in seq.split(",")]
        for e in experts[:-1]:
            ensure_slots(st, 0, [e], False)
        before = st.slot_key.copy()
        ms, mk = ensure_slots(st, 0, [experts[-1]], False)
        assert ms == [int(victim)] and before[int(victim)] == int(evicted) and mk == [experts[-1]]


def _lrfu_by_definition(lam, refs, t):
    """C(t) = sum over references t_i of 2^(-lam (t - t_i)), in fp64, from the
    full reference list (the published definition, no incremental update)."""
    return sum(2.0 ** (-lam * (t - ti)) for ti in refs)


def test_incremental_fixed_point_lrfu_follows_the_definition():
    # random chunks of one or two queries of one to three experts; whenever
    # the definition's smallest candidate value is clear of the next by more
    # than the fixed point's error, the oracle's victim is that candidate
    g = np.random.default_rng(1)
    for lam_inv, D in ((2, HALF), (8, 3938502375), (64, 4248701964)):
        assert abs(D / 2 ** 32 - 2.0 ** (-1.0 / lam_inv)) < 2 ** -31
        S, E = 6, 20
        st = _bank(S, E, POLICY_LRFU, D)
        refs = {}                       # key -> reference times since admission
        checked = 0
        for chunk in range(150):
            nq = int(g.integers(1, 3))
            for q in range(nq):
                width = int(g.integers(1, 4))
                query = sorted(set(int(min(E - 1, g.zipf(1.4) - 1)) for _ in range(width)))
                t = st.clock + 1
                pin = t if q == 0 else st.chunk_start
                hits = [e for e in query if st.key_to_slot[e] >= 0]
                misses = [e for e in query if st.key_to_slot[e] < 0]
                for e in hits:
                    refs[e].append(t)
                cand = []
                for s in range(S):
                    k = int(st.slot_key[s])
                    if int(st.slot_stamp[s]) < pin and k not in hits:      # this query's hits are touched first
                        cand.append((_lrfu_by_definition(1.0 / lam_inv, refs.get(k, []), t) if k >= 0 else 0.0, s))
                cand.sort()
                ms, mk = ensure_slots(st, 0, query, False, chunk_first=(q == 0))
                for i, (slot, key) in enumerate(zip(ms, mk)):
                    clear = i + 1 >= len(cand) or cand[i + 1][0] - cand[i][0] > 1e-5 * max(1.0, cand[i][0])
                    clear = clear and (i == 0 or cand[i][0] - cand[i - 1][0] > 1e-5 * max(1.0, cand[i][0]))
                    if clear:
                        assert slot == cand[i][1], (lam_inv, chunk, q, i)
                        checked += 1
                    refs[key] = [t]
                for k in list(refs):
                    if st.key_to_slot[k] < 0:
                        del refs[k]
        assert checked > 50, checked


def test_small_lambda_evicts_the_least_referenced():
    # lambda = 1/4096 over 60 ticks: a reference counts 0.99 or more, so a
    # candidate with fewer references always has the smaller value
    g = np.random.default_rng(3)
    D = 4294240539                   # floor(2^32 * 2^(-1/4096))
    S, E = 5, 16
    st = _bank(S, E, POLICY_LRFU, D)
    count = {}
    for t in range(60):
        e = int(min(E - 1, g.zipf(1.3) - 1))
        if st.key_to_slot[e] >= 0:
            ensure_slots(st, 0, [e], True)
            count[e] += 1
            continue
        cand = [count.get(int(st.slot_key[s]), 0) if st.slot_key[s] >= 0 else 0 for s in range(S)]
        ms, _ = ensure_slots(st, 0, [e], True)
        assert cand[ms[0]] == min(cand), t
        count = {k: v for k, v in count.items() if st.key_to_slot[k] >= 0}
        count[e] = 1


def test_lambda_one_orders_like_lru_over_short_histories():
    # lambda = 1: the last reference outweighs all earlier ones (2^-d >
    # sum over i > d of 2^-i), so with one expert per query and at most 24
    # ticks of history the victims are LRU's
    g = np.random.default_rng(2)
    S, E = 5, 9
    a, b = _bank(S, E, POLICY_LRFU, LAMBDA1), _bank(S, E, POLICY_LRU, 0)
    for t in range(20):
        e = int(g.integers(0, E))
        assert ensure_slots(a, 0, [e], True) == ensure_slots(b, 0, [e], True), t
    assert np.array_equal(a.slot_key, b.slot_key)


def test_a_chunk_never_evicts_its_own_earlier_admissions():
    # a frequently used expert 9 sits in slot 0; the chunk's first query admits
    # expert 1 (value 1.0, lower than expert 9's); the second query's miss must
    # not take expert 1's slot (pinned), although its value is the smallest
    st = _bank(3, 12, POLICY_LRFU, HALF)
    for _ in range(4):
        ensure_slots(st, 0, [9], True)
    ensure_slots(st, 0, [8], True)                       # slot 1
    ms1, _ = ensure_slots(st, 0, [1], True)              # chunk start: slot 2 (empty)
    assert ms1 == [2]
    ms2, _ = ensure_slots(st, 0, [2], False)             # same chunk
    assert ms2 != [2] and st.key_to_slot[1] == 2
    # the same second query as a chunk of its own may evict expert 1
    st2 = _bank(3, 12, POLICY_LRFU, HALF)
    for _ in range(4):
        ensure_slots(st2, 0, [9], True)
    ensure_slots(st2, 0, [8], True)
    ensure_slots(st2, 0, [1], True)
    ms3, _ = ensure_slots(st2, 0, [2], True)
    assert ms3 == [1] or ms3 == [2]
