"""LRU slot bank keyed by (layer, expert) (oracle).

Sources:
  * FreeToken PR #676, "Problem" and "Solution": in decode, only routed
    experts are brought in through the slot cache; a short prefill chunk
    feeds its distinct experts to the LRU in slices of fixed width, moves
    every slice's misses in before the following slice is queried, and
    records none of these admissions in the decode counters or the LRU
    statistics.
  * Same page, author's reply: eviction there is plain LRU, which never
    picks a slice admitted earlier in the chunk while older slots remain,
    so no pinning is needed; one layer's expert set always fits in the
    cache.
  * vLLM fork PR #48, "What": one bank shared by all MoE layers, keyed
    (layer, expert), planned by an LRU over the bank.

Readings taken where the pages are silent (each one is a stated choice):
  1. one recency stamp per query (the clock ticks once per call, also for a
     query holding only sentinels); ties between equal stamps go to the
     lower slot index;
  2. a never-used slot has stamp 0, so empty slots are taken first, lowest
     index first;
  3. hits are touched before victims are chosen, so a query never evicts its
     own hits;
  4. the i-th miss (query order) takes the i-th candidate in ascending
     (stamp, slot); candidates are the slots not stamped by this query;
  5. with record_stats off the recency stamps still move (only the
     statistics stay untouched);
  6. a miss with no candidate left sets the capacity error bit and is not
     admitted.
key = layer * E + expert.

Scored eviction (LRFU).  Sources: FreeToken PR #676, the run notes (the
author's own build admits by LRFU rather than LRU) and "Solution" (with a
scored eviction policy the earlier pieces' slots also need pinning against
the later ones).  The pages name the policy only; its definition here is the
published LRFU (Lee et al., "LRFU: a spectrum of policies that subsumes the
LRU and LFU policies"): a slot's combined recency-frequency value is
C(t) = sum over its references t_i since admission of 2^(-lambda (t - t_i)),
kept as C at the last reference L and decayed to the present as
C(L) * 2^(-lambda (t - L)); the victim is the smallest present value.
Readings (stated choices, all integer so that every decision is exact):
  7. C is unsigned Q8.24 fixed point (1.0 = 2^24), saturating at 2^32 - 1;
     the decay per tick is a caller-given Q0.32 factor D = 2^32 * 2^-lambda
     (an input, 0 < D < 2^32), raised to the n-th power by right-to-left
     binary exponentiation with truncation after each product, starting from
     1.0 = 2^32: r = 2^32, b = D; for each bit of n from the lowest: if set,
     r = r * b >> 32; then b = b * b >> 32;
     decay(C, n) = C * r >> 32;
  8. a hit: C = min(decay(C, now - L) + 1.0, 2^32 - 1), L = now; an
     admission: C = 1.0, L = now; the stamp is L, as for LRU;
  9. candidates are the slots untouched by the whole chunk (stamp below the
     clock of the chunk's first query: the pin), ordered by (decay(C, now -
     L), slot); a chunk starts with the query at q_begin = 0 (per-query
     calls) or with the first query of one batched call;
 10. the LRU rules 1-6 stand otherwise; under LRU nothing is pinned beyond
     rule 4 (the pages' author: LRU evicts the earlier queries last).

Parity: pinned (page-printed query splits 128+32 and 3+3+2, statistics
untouched by prefill, earlier queries evicted last, agreement with a textbook
recency-list LRU whenever stamps are distinct, bijection invariant; LRFU:
exact-rational bounds on the fixed-point power, the LFU limit against a
textbook least-frequently-used order, the LRU limit, pinning against a
chunk's own admissions, a hand-worked example in tests/golden).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

ERR_CAPACITY = 1

STAT_HITS, STAT_MISSES, STAT_EVICTIONS, STAT_QUERIES = range(4)

POLICY_LRU, POLICY_LRFU = 0, 1
CRF_ONE = 1 << 24
CRF_MAX = (1 << 32) - 1


def pow_q32(D: int, n: int) -> int:
    """D^n in Q0.32 by right-to-left binary exponentiation, truncating each
    product (reading 7); 1.0 = 2^32 for n = 0."""
    r, b = 1 << 32, int(D)
    n = int(n)
    while n > 0:
        if n & 1:
            r = (r * b) >> 32
        b = (b * b) >> 32
        n >>= 1
    return r


def crf_decay(c: int, n: int, D: int) -> int:
    """A Q8.24 value decayed over n ticks."""
    return (int(c) * pow_q32(D, n)) >> 32


@dataclass
class SlotBankState:
    S: int
    L: int
    E: int
    slot_key: np.ndarray = None      # int32 [S], -1 empty
    slot_stamp: np.ndarray = None    # uint64 [S], 0 never used
    key_to_slot: np.ndarray = None   # int32 [L*E], -1 not resident
    clock: int = 0
    stats: np.ndarray = None         # uint64 [4]
    decode_freq: np.ndarray = None   # uint32 [L*E]
    err: int = 0
    policy: int = POLICY_LRU
    decay_q32: int = 0               # LRFU: per-tick decay factor D (Q0.32)
    slot_crf: np.ndarray = None      # uint32 [S], LRFU value at the slot's stamp (Q8.24)
    chunk_start: int = 0             # clock of the current chunk's first query

    def __post_init__(self):
        if self.slot_key is None:
            self.slot_key = np.full(self.S, -1, np.int32)
        if self.slot_stamp is None:
            self.slot_stamp = np.zeros(self.S, np.uint64)
        if self.key_to_slot is None:
            self.key_to_slot = np.full(self.L * self.E, -1, np.int32)
            for s in range(self.S):
                if self.slot_key[s] >= 0:
                    self.key_to_slot[self.slot_key[s]] = s
        if self.stats is None:
            self.stats = np.zeros(4, np.uint64)
        if self.decode_freq is None:
            self.decode_freq = np.zeros(self.L * self.E, np.uint32)
        if self.slot_crf is None:
            self.slot_crf = np.zeros(self.S, np.uint32)

    @classmethod
    def from_fill(cls, fill):
        st = cls(fill.S, fill.L, fill.E, fill.slot_key.copy(), fill.slot_stamp.copy())
        st.clock = int(fill.clock)
        return st

    def copy(self):
        c = SlotBankState(self.S, self.L, self.E, self.slot_key.copy(), self.slot_stamp.copy(),
                          self.key_to_slot.copy(), self.clock, self.stats.copy(),
                          self.decode_freq.copy(), self.err, self.policy, self.decay_q32,
                          self.slot_crf.copy(), self.chunk_start)
        return c


def ensure_slots(st: SlotBankState, layer: int, query, record_stats: bool, chunk_first: bool = True):
    """Admit one query of expert ids of ``layer``; mutates ``st``.

    ``chunk_first``: this query starts a chunk (LRFU pins every slot the
    chunk touches from here on; LRU ignores it).
    Returns (miss_slot list, miss_key list): the admitted misses in query
    order, whose host rows the caller copies into the listed slots before
    the next query.
    """
    st.clock += 1
    now = st.clock
    if chunk_first:
        st.chunk_start = now
    E = st.E
    lrfu = st.policy == POLICY_LRFU
    keys = [layer * E + int(e) for e in query if 0 <= int(e) < E]
    hits, misses = [], []
    for key in keys:
        s = int(st.key_to_slot[key])
        if s >= 0:
            hits.append((key, s))
        else:
            misses.append(key)
    for _, s in hits:
        if lrfu:
            c = crf_decay(int(st.slot_crf[s]), now - int(st.slot_stamp[s]), st.decay_q32) + CRF_ONE
            st.slot_crf[s] = min(c, CRF_MAX)
        st.slot_stamp[s] = now
    if lrfu:
        pin = st.chunk_start
        cand = sorted((crf_decay(int(st.slot_crf[s]), now - int(st.slot_stamp[s]), st.decay_q32), s)
                      for s in range(st.S) if int(st.slot_stamp[s]) < pin)
    else:
        cand = sorted((int(st.slot_stamp[s]), s) for s in range(st.S) if int(st.slot_stamp[s]) < now)
    miss_slot, miss_key = [], []
    evicted = 0
    for i, key in enumerate(misses):
        if i >= len(cand):
            st.err |= ERR_CAPACITY
            continue
        s = cand[i][1]
        old = int(st.slot_key[s])
        if old >= 0:
            st.key_to_slot[old] = -1
            evicted += 1
        st.slot_key[s] = key
        st.key_to_slot[key] = s
        st.slot_stamp[s] = now
        if lrfu:
            st.slot_crf[s] = CRF_ONE
        miss_slot.append(s)
        miss_key.append(key)
    if record_stats:
        st.stats[STAT_HITS] += len(hits)
        st.stats[STAT_MISSES] += len(miss_key)
        st.stats[STAT_EVICTIONS] += evicted
        st.stats[STAT_QUERIES] += 1
        for key in keys:
            st.decode_freq[key] += 1
    return miss_slot, miss_key
