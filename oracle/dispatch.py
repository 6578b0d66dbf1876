"""Host-side dispatch predicates (oracle).

Sources: FreeToken PR #676, "Solution" and "Tests": a threshold N of 0 takes
no chunk on demand; otherwise a chunk of at most N tokens takes the demand
path (96 tokens do at N = 96, 97 tokens stream; N = 2 takes 1 and 2 tokens).
Same page, author's reply: the expert set of one layer always fits in the
cache (the capacity guard below).  gdevenyi's PR #68, second commit: a layer needing more than
half the cache takes the whole-layer path.

Parity: pinned (the page-printed threshold cases).
"""


def prefill_on_demand(T: int, threshold: int) -> bool:
    return threshold > 0 and 0 < T <= threshold


def demand_capacity_ok(T: int, k: int, E: int, S: int, half: bool = False) -> bool:
    need = min(T * k, E)
    return need <= (S // 2 if half else S)
