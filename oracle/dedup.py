"""Distinct-expert list (oracle).

Source: FreeToken PR #676, "Solution" (the LRU receives the chunk's distinct
experts as an ordered list whose length the host knows in advance, which is
what spares a host synchronisation) and gdevenyi's comment there (the LRU
gets unique ids only; routes find their entry again through the inverse
index of the unique operation).

Reading taken: the fixed length is min(n, E) (the largest possible distinct
count, known to the host); unused tail entries hold the sentinel E; ids
outside [0, E) are not experts and are ignored (their inverse is -1).

Parity: pinned (Python set/sorted cross-check, page-printed count of 160).
"""
import numpy as np


def dedup_sorted(ids: np.ndarray, E: int):
    """ids int [n] -> (distinct int32 [min(n,E)], n_distinct, inverse int32 [n])."""
    ids = np.asarray(ids).reshape(-1)
    n = ids.size
    lmax = min(n, E)
    valid = (ids >= 0) & (ids < E)
    uniq = np.unique(ids[valid])
    distinct = np.full(lmax, E, dtype=np.int32)
    distinct[:uniq.size] = uniq
    inverse = np.full(n, -1, dtype=np.int32)
    inverse[valid] = np.searchsorted(uniq, ids[valid]).astype(np.int32)
    return distinct, int(uniq.size), inverse
