"""Align routes into fixed-size per-bucket blocks (oracle).

Sources: FreeToken PR #676, "Solution" (a demand chunk is aligned over the
bank's slots, so bucket counts beyond 1023 must work) and "Tests" (the align
test places each route exactly one time, inside a block owned by the route's
expert, for 1023 and for 2100 experts); gdevenyi's comment there (an align
without the one-block limit checked at 2100 and 4096 buckets);
vLLM fork PR #48, "What" (align over logical experts ignoring invalid
ones, then remap to physical rows).

Readings taken:
  * bucket of route r = id_to_bucket[ids[r]] when a map is given, else ids[r];
    routes whose id or bucket is out of range are dropped;
  * inside a bucket, routes keep ascending route index (the pages only say
    outputs are identical across aligners; a fixed order is what makes the
    grouped GEMM reproducible);
  * each bucket's count c is padded to ceil(c / B) * B with the sentinel n
    (the route count); buckets are laid out in ascending bucket order;
  * block j of the padded list belongs to bucket block_bucket[j]; entries
    past the padded total hold sentinel n and block id -1;
  * the active-bucket list holds the non-empty buckets in ascending order
    with the first block index of each (plus a final end entry).

Parity: pinned (page invariant at 1023/1024/2100/4096 buckets, brute-force
placement on tiny inputs, stable-argsort closed form).
"""
import numpy as np


def align_capacity(n: int, num_buckets: int, B: int) -> int:
    """Length of the padded route list: n + min(n, Nb) * (B - 1), rounded up to B."""
    cap = n + min(n, num_buckets) * (B - 1)
    return ((cap + B - 1) // B) * B


def align_blocks(ids: np.ndarray, id_to_bucket, num_buckets: int, B: int):
    ids = np.asarray(ids).reshape(-1).astype(np.int64)
    n = ids.size
    if id_to_bucket is not None:
        m = np.asarray(id_to_bucket).astype(np.int64)
        ok = (ids >= 0) & (ids < m.size)
        bucket = np.full(n, -1, np.int64)
        bucket[ok] = m[ids[ok]]
    else:
        bucket = ids.copy()
    valid = (bucket >= 0) & (bucket < num_buckets)
    cap = align_capacity(n, num_buckets, B)
    sorted_routes = np.full(cap, n, np.int32)
    block_bucket = np.full(cap // B, -1, np.int32)
    per_bucket = [[] for _ in range(num_buckets)]
    for r in range(n):                       # ascending route index
        if valid[r]:
            per_bucket[int(bucket[r])].append(r)
    active, begin = [], []
    pos = 0
    for b in range(num_buckets):
        routes = per_bucket[b]
        c = len(routes)
        if c == 0:
            continue
        padded = -(-c // B) * B
        sorted_routes[pos:pos + c] = routes
        block_bucket[pos // B:(pos + padded) // B] = b
        active.append(b)
        begin.append(pos // B)
        pos += padded
    begin.append(pos // B)
    return {
        "sorted_routes": sorted_routes,
        "block_bucket": block_bucket,
        "n_post_pad": pos,
        "active_buckets": np.array(active, np.int32),
        "active_block_begin": np.array(begin, np.int32),
        "n_active": len(active),
        "capacity": cap,
    }
