"""GPU parity of the one-launch chunk planner: dedup + all LRU queries + align
in one workgroup gives exactly the outputs, bank state and copied rows of the
separate calls, and (through them) of the oracle's LRU."""
import numpy as np
import pytest
import torch

import workloads as W
from helpers import ExpertSource, fill_pool, flush
from oracle import SlotBankState, ensure_slots

pytestmark = pytest.mark.gpu

# outputs written in full; active_buckets / active_block_begin are defined up
# to n_active / n_active + 1 entries (the rest of those buffers is not written)
OUT_KEYS = ("distinct", "n_distinct", "n_miss", "n_total", "sorted_routes", "block_bucket", "n_post_pad",
            "n_active")
STATE_KEYS = ("slot_key", "slot_stamp", "key_to_slot", "clock", "stats", "decode_freq", "err")


def _plan_both(S, NL, E, k, T, logits, fill, width, record_stats, layer=0, rec=4096, seed=11, ids=None):
    """Runs the separate calls and the fused planner from the same bank state;
    returns both (buffers, bank) pairs.  ``ids`` (T, k) replaces routing the
    logits (for expert counts beyond the router's limit)."""
    import slot_cache_routed_amd.layer as LY
    import slot_cache_routed_amd._lib as L
    pool = LY.HostPool(NL, E, rec, E, payload_of=lambda key: key % E)
    g = np.random.default_rng(seed)
    for p in range(E):
        pool.write_payload(p, g.integers(0, 256, size=rec, dtype=np.uint8))
    dev = None if ids is not None else torch.from_numpy(np.ascontiguousarray(logits)).cuda()
    s = torch.cuda.current_stream().cuda_stream
    out = []
    for fused in (False, True):
        bank = LY.Bank(S, NL, E, 0, rec)
        if fill is not None:
            bank.load_fill(fill)
        buf = LY.LayerBuffers(T, E, k, 128, 128, S, 0, width=width)
        if ids is None:
            L.route(dev, T, E, k, buf["topk_ids"], buf["topk_w"], s)
        else:
            buf["topk_ids"].copy_(torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).reshape(-1))
        if fused:
            assert LY.plan(buf, bank, pool, layer, record_stats)
        else:
            L.dedup(buf["topk_ids"], buf.R, E, buf["distinct"], buf["n_distinct"], buf["inverse"], s)
            LY.admit(buf, bank, pool, layer, record_stats, batched=True)
            LY.align(buf, bank.key_to_slot.data_ptr() + layer * E * 4, E)
        torch.cuda.synchronize()
        out.append((buf, bank))
    return out


def _compare(out, where):
    (b0, k0), (b1, k1) = out
    for key in OUT_KEYS:
        assert torch.equal(b0[key], b1[key]), (where, key)
    na = int(b0["n_active"].item())
    assert torch.equal(b0["active_buckets"][:na], b1["active_buckets"][:na]), where
    assert torch.equal(b0["active_block_begin"][:na + 1], b1["active_block_begin"][:na + 1]), where
    nt = int(b0["n_total"].item())
    assert torch.equal(b0["miss_slot"][:nt], b1["miss_slot"][:nt]) and torch.equal(b0["miss_key"][:nt],
                                                                                   b1["miss_key"][:nt]), where
    s0, s1 = k0.snapshot(), k1.snapshot()
    for key in STATE_KEYS:
        assert np.array_equal(np.asarray(s0[key]), np.asarray(s1[key])), (where, key)
    assert torch.equal(k0.rows, k1.rows), (where, "bank rows")
    return s1


def test_plan_short_prefill_96_equals_separate_calls():
    cfg = W.C2
    E, k, S, NL, T = cfg.shape.E, cfg.shape.k, cfg.S, cfg.L, cfg.T
    lg, _ = W.logits_with_chosen(cfg.seed, T, E, k, 160)
    fill = W.bank_prefilled(cfg.seed, S, NL, E, 600, exclude_layer=0)
    out = _plan_both(S, NL, E, k, T, lg, fill, 128, False, rec=1024)
    _compare(out, "short prefill")
    assert out[1][0]["n_miss"].cpu().numpy().tolist() == [128, 32, 0, 0]
    flush("plan: 96-token chunk equals the separate calls")


def test_plan_one_layer_cache_three_per_query():
    cfg = W.C3B
    E, k, T = cfg.shape.E, cfg.shape.k, cfg.T
    lg = W.logits_normal(cfg.seed, 0, T, E)
    fill = W.bank_prefilled(cfg.seed, 8, cfg.L, E, 8, exclude_layer=0)
    out = _plan_both(8, cfg.L, E, k, T, lg, fill, 3, False, rec=512)
    _compare(out, "S=8 W=3")
    assert out[1][0]["n_miss"].cpu().numpy().tolist() == [3, 3, 2]


@pytest.mark.parametrize("S,E,k,T,width,stats", [(6, 16, 3, 40, 4, 0), (30, 64, 4, 50, 16, 1), (700, 512, 10, 12, 32, 1)])
def test_plan_small_banks_overflow_and_decode(S, E, k, T, width, stats):
    # S=6 with up to 16 distinct: later queries take earlier slots again (superseded
    # entries) and overflow the bank (error bit); the others are decode-like chunks
    g = np.random.default_rng(S + E)
    lg = g.standard_normal((T, E)).astype(np.float32)
    out = _plan_both(S, 2, E, k, T, lg, None, width, stats, layer=1, rec=512)
    snap = _compare(out, f"S={S} E={E}")
    # the bank state also equals the oracle's LRU run query by query
    from oracle import route_topk_softmax, dedup_sorted
    ids, _ = route_topk_softmax(lg, k)
    distinct, _, _ = dedup_sorted(ids.reshape(-1), E)
    st = SlotBankState(S, 2, E)
    for q0 in range(0, len(distinct), width):
        ensure_slots(st, 1, distinct[q0:q0 + width], bool(stats))
    for key in ("slot_key", "slot_stamp", "key_to_slot", "clock", "stats", "decode_freq", "err"):
        assert np.array_equal(np.asarray(snap[key]), np.asarray(getattr(st, key))), key


def test_plan_reports_unsupported_shapes_without_launching():
    import slot_cache_routed_amd.layer as LY
    import slot_cache_routed_amd._lib as L
    S, E, k, T = 9000, 16, 2, 4     # more slots than the one-workgroup align takes
    bank = LY.Bank(S, 1, E, 0, 256)
    buf = LY.LayerBuffers(T, E, k, 128, 128, S, 0, width=8)
    pool = LY.HostPool(1, E, 256, E)
    before = bank.snapshot()
    assert not LY.plan(buf, bank, pool, 0, False)
    torch.cuda.synchronize()
    after = bank.snapshot()
    assert after["clock"] == before["clock"]


def test_plan_at_its_largest_shape_against_the_oracle():
    # 4096 routes, 8192 experts, 8192 slots, queries of 1024: the one-workgroup
    # limits of the planner, with evictions (more distinct experts than free slots)
    S, E, k, T, width = 8192, 8192, 8, 512, 1024
    g = np.random.default_rng(8192)
    ids = np.stack([g.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    fill = W.bank_prefilled(3, S, 2, E, 6000, exclude_layer=1)
    out = _plan_both(S, 2, E, k, T, None, fill, width, 1, layer=1, rec=256, ids=ids)
    snap = _compare(out, "largest")
    from oracle import dedup_sorted
    distinct, nd, _ = dedup_sorted(ids.reshape(-1), E)
    st = SlotBankState.from_fill(fill)
    for q0 in range(0, len(distinct), width):
        ensure_slots(st, 1, distinct[q0:q0 + width], True)
    for key in ("slot_key", "slot_stamp", "key_to_slot", "clock", "stats", "decode_freq", "err"):
        assert np.array_equal(np.asarray(snap[key]), np.asarray(getattr(st, key))), key
    flush(f"plan at 4096 routes / 8192 experts / 8192 slots: {nd} distinct")


@pytest.mark.parametrize("planner", ["batched", "plan_chunk"])
@pytest.mark.parametrize("stats", [0, 1])
@pytest.mark.parametrize("policy", ["lru", "lrfu"])
def test_all_hit_chunks_against_the_oracle(policy, stats, planner):
    """A chunk whose experts are all resident admits nothing, and the planners
    then touch every hit without selecting candidates.  Three chunks of layer
    1: one that admits its experts, the same chunk again (all hits), and a
    chunk of a subset of them (all hits, more trailing queries of sentinels).
    After each, the bank state (stamps at each query's own clock, the LRFU
    values, counts, frequencies, clock) and the per-query miss counts equal
    the oracle's query-by-query run."""
    import math
    import slot_cache_routed_amd.layer as LY
    import slot_cache_routed_amd._lib as L
    from oracle import dedup_sorted
    from oracle.lru import POLICY_LRFU
    S, E, NL, k, T, width, rec, layer = 200, 128, 2, 4, 30, 16, 256, 1
    D = math.floor(2 ** 32 * 2 ** (-1.0 / 4))
    pol = L.SCR_POLICY_LRFU if policy == "lrfu" else L.SCR_POLICY_LRU
    g = np.random.default_rng(77)
    ids = np.stack([g.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    chunks = [ids, ids, ids[:9]]
    pool = LY.HostPool(NL, E, rec, E, payload_of=lambda key: key % E)
    fill = W.bank_prefilled(5, S, NL, E, 120, exclude_layer=layer)
    bank = LY.Bank(S, NL, E, 0, rec, policy=pol, lrfu_decay=D)
    bank.load_fill(fill)
    st = SlotBankState.from_fill(fill)
    if policy == "lrfu":
        st.policy, st.decay_q32 = POLICY_LRFU, D
    s = torch.cuda.current_stream().cuda_stream
    for c, chunk in enumerate(chunks):
        Tc = chunk.shape[0]
        buf = LY.LayerBuffers(Tc, E, k, 128, 128, S, 0, width=width)
        buf["topk_ids"].copy_(torch.from_numpy(np.ascontiguousarray(chunk)).reshape(-1))
        if planner == "plan_chunk":
            assert LY.plan(buf, bank, pool, layer, bool(stats))
        else:
            L.dedup(buf["topk_ids"], buf.R, E, buf["distinct"], buf["n_distinct"], buf["inverse"], s)
            LY.admit(buf, bank, pool, layer, bool(stats), batched=True)
        torch.cuda.synchronize()
        distinct, nd, _ = dedup_sorted(chunk.reshape(-1), E)
        misses = []
        for q0 in range(0, len(distinct), width):
            ms, _ = ensure_slots(st, layer, distinct[q0:q0 + width], bool(stats), chunk_first=(q0 == 0))
            misses.append(len(ms))
        assert buf["n_miss"].cpu().numpy()[:len(misses)].tolist() == misses, (c, misses)
        assert (sum(misses) == 0) == (c > 0), c
        snap = bank.snapshot()
        for key in ("slot_key", "slot_stamp", "key_to_slot", "clock", "stats", "decode_freq", "err", "slot_crf"):
            assert np.array_equal(np.asarray(snap[key]), np.asarray(getattr(st, key))), (c, key)
    flush(f"all-hit chunks ({policy}, stats {stats}, {planner}): bank state equals the oracle")


@pytest.mark.parametrize("i", range(8))
def test_seeded_chains_of_chunks_against_the_oracle(i):
    """One bank through 24 chunks of Zipf-skewed routing over its layers, each
    planned in one launch: bank state (LRU or LRFU, decode counters on or off,
    capacity errors included) bit-exact against the oracle's query-by-query
    admission after every chunk, and resident rows equal to their records."""
    import math
    import slot_cache_routed_amd._lib as L
    import slot_cache_routed_amd.layer as LY
    from oracle import dedup_sorted, route_topk_softmax
    from oracle.lru import POLICY_LRFU
    r = np.random.default_rng(60000 + i)
    E = int(r.choice([8, 16, 64, 256, 512]))
    k = int(r.integers(1, min(E, 10) + 1))
    T = min(int(r.choice([1, 4, 16, 96, 300])), 4096 // k)
    NL = int(r.choice([1, 2, 4]))
    S = int(r.choice([k + 2, 16, 64, 200, 1100]))
    width = int(r.choice([w for w in (1, 4, 16, 32, 128) if w <= S]))
    lrfu, stats = i % 2 == 1, bool(r.integers(0, 2))
    D = math.floor(2 ** 32 * 2 ** (-1.0 / int(r.choice([2, 16, 64]))))
    flush(f"chain {i}: S={S} E={E} k={k} T={T} layers={NL} width={width} lrfu={lrfu} stats={stats}")
    rec = 512
    pool = LY.HostPool(NL, E, rec, E, payload_of=lambda key: key % E)
    g = np.random.default_rng(60000 + i)
    for p in range(E):
        pool.write_payload(p, g.integers(0, 256, size=rec, dtype=np.uint8))
    if lrfu:
        bank = LY.Bank(S, NL, E, 0, rec, policy=L.SCR_POLICY_LRFU, lrfu_decay=D)
    else:
        bank = LY.Bank(S, NL, E, 0, rec)
    st = SlotBankState(S, NL, E)
    if lrfu:
        st.policy, st.decay_q32 = POLICY_LRFU, D
    buf = LY.LayerBuffers(T, E, k, 128, 128, S, 0, width=width)
    s = torch.cuda.current_stream().cuda_stream
    for step in range(24):
        layer = step % NL
        lg = W.zipf_gumbel_logits(60000 + i, layer, step, T, E)
        L.route(torch.from_numpy(np.ascontiguousarray(lg)).cuda(), T, E, k, buf["topk_ids"], buf["topk_w"], s)
        assert LY.plan(buf, bank, pool, layer, stats)
        torch.cuda.synchronize()
        ids, _ = route_topk_softmax(lg, k)
        distinct, _, _ = dedup_sorted(ids.reshape(-1), E)
        for q0 in range(0, len(distinct), width):
            ensure_slots(st, layer, distinct[q0:q0 + width], stats, chunk_first=(q0 == 0))
        snap = bank.snapshot()
        for key in STATE_KEYS:
            assert np.array_equal(np.asarray(snap[key]), np.asarray(getattr(st, key))), (step, key)
        if lrfu:
            assert np.array_equal(np.asarray(snap["slot_crf"]), np.asarray(st.slot_crf)), (step, "slot_crf")
        if int(np.asarray(snap["err"])) == 0:
            rows = bank.rows.view(S, -1).cpu().numpy()
            for slot in np.nonzero(np.asarray(snap["slot_key"]) >= 0)[0]:
                key = int(np.asarray(snap["slot_key"])[slot])
                assert np.array_equal(rows[slot], pool.key_record(key).numpy()), (step, "row", slot)
    hits, misses, ev, _ = [int(v) for v in st.stats]
    flush(f"chain {i}: hits {hits} misses {misses} evictions {ev} err {int(np.asarray(st.err))}")
