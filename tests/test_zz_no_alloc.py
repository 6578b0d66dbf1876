"""The entry point that allocates nothing (scr_align_blocks_noalloc, for
callers that cannot allocate device memory): through the C ABI, two calls in
a row, the second on a smaller input, each against scr_align_blocks with its
own workspace (bit-exact) and the second also against the oracle.  Both
inputs take the multi-workgroup align, the one that uses the scratch array,
and the second runs on the array the first left behind."""
import numpy as np
import pytest
import torch

import workloads as W
from helpers import flush
from oracle import align_blocks

pytestmark = pytest.mark.gpu


def _outputs(n, nb, B):
    import slot_cache_routed_amd._lib as L
    cap = L.align_capacity(n, nb, B)
    m = min(n, nb)
    return cap, {
        "sorted_routes": torch.full((cap,), -7, dtype=torch.int32, device="cuda"),
        "block_bucket": torch.full((cap // B,), -7, dtype=torch.int32, device="cuda"),
        "n_post_pad": torch.full((1,), -7, dtype=torch.int32, device="cuda"),
        "active_buckets": torch.full((m,), -7, dtype=torch.int32, device="cuda"),
        "active_block_begin": torch.full((m + 1,), -7, dtype=torch.int32, device="cuda"),
        "n_active": torch.full((1,), -7, dtype=torch.int32, device="cuda"),
    }


def _host(out, cap, B):
    h = {k: v.cpu().numpy() for k, v in out.items()}
    na = int(h["n_active"][0])
    return {"sorted_routes": h["sorted_routes"][:cap], "block_bucket": h["block_bucket"][:cap // B],
            "n_post_pad": int(h["n_post_pad"][0]), "n_active": na, "active_buckets": h["active_buckets"][:na],
            "active_block_begin": h["active_block_begin"][:na + 1]}


KEYS = ("sorted_routes", "block_bucket", "active_buckets", "active_block_begin")


@pytest.mark.parametrize("first,second", [((300000, 2100, 16, None), (50000, 1023, 64, 700))])
def test_noalloc_align_equals_the_workspace_align_twice(first, second):
    import slot_cache_routed_amd._lib as L
    s = torch.cuda.current_stream().cuda_stream
    g = np.random.default_rng(42)
    for n, nb, B, n_map in (first, second):
        flush(f"no-alloc align: n={n} buckets={nb} block={B} map={n_map}")
        if n_map is None:
            ids = W.uniform_ids(4, n, nb).astype(np.int32)
            ids[::97] = nb + 3                                   # invalid buckets are dropped
            id_map = None
        else:
            ids = g.integers(-2, n_map + 2, size=n).astype(np.int32)   # some ids outside the map
            id_map = g.integers(-1, nb, size=n_map).astype(np.int32)   # some unmapped ids
        d_ids = torch.from_numpy(ids).cuda()
        d_map = None if id_map is None else torch.from_numpy(id_map).cuda()
        num_ids = 0 if id_map is None else n_map
        cap, ref = _outputs(n, nb, B)
        ws = torch.empty(L.align_workspace(n, nb), dtype=torch.uint8, device="cuda")
        L.align_blocks(d_ids, n, d_map, num_ids, nb, B, *[ref[k] for k in ("sorted_routes", "block_bucket",
                       "n_post_pad", "active_buckets", "active_block_begin", "n_active")], ws, ws.numel(), s)
        _, got = _outputs(n, nb, B)
        L.align_blocks_noalloc(d_ids, n, d_map, num_ids, nb, B, *[got[k] for k in ("sorted_routes", "block_bucket",
                               "n_post_pad", "active_buckets", "active_block_begin", "n_active")], s)
        torch.cuda.synchronize()
        r, o = _host(ref, cap, B), _host(got, cap, B)
        assert o["n_post_pad"] == r["n_post_pad"] and o["n_active"] == r["n_active"]
        for k in KEYS:
            assert np.array_equal(o[k], r[k]), k
        if n_map is not None:
            want = align_blocks(ids, id_map, nb, B)
            assert o["n_post_pad"] == want["n_post_pad"] and o["n_active"] == want["n_active"]
            for k in KEYS:
                assert np.array_equal(o[k], np.asarray(want[k])), ("oracle", k)
        flush(f"no-alloc align: n={n}: {o['n_active']} active buckets, {o['n_post_pad']} padded routes, equal")
