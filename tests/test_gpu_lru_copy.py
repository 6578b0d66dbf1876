"""GPU parity: the LRU planner (bit-exact bank state after every query) and
the fixed-grid miss copy (bank rows byte-equal to the pinned host records)."""
import numpy as np
import pytest
import torch

import workloads as W
from conftest import read_golden
from helpers import flush
from oracle import SlotBankState, dedup_sorted, ensure_slots, route_topk_softmax

pytestmark = pytest.mark.gpu


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _bank(S, n_layers, E, rec=256):
    import slot_cache_routed_amd.layer as LY
    return LY.Bank(S, n_layers, E, 0, rec)


def _same_state(bank, st, where=""):
    snap = bank.snapshot()
    assert np.array_equal(snap["slot_key"], st.slot_key), where
    assert np.array_equal(snap["slot_stamp"], st.slot_stamp), where
    assert np.array_equal(snap["key_to_slot"], st.key_to_slot), where
    assert snap["clock"] == st.clock, where
    assert np.array_equal(snap["stats"], st.stats), where
    assert np.array_equal(snap["decode_freq"], st.decode_freq), where
    assert snap["err"] == st.err, where


class _Q:
    def __init__(self, width):
        self.ms = torch.full((width,), -1, dtype=torch.int32, device="cuda")
        self.mk = torch.full((width,), -1, dtype=torch.int32, device="cuda")
        self.nm = torch.full((1,), -1, dtype=torch.int32, device="cuda")


def _ensure_gpu(bank, layer, dist_dev, q0, width, record):
    import slot_cache_routed_amd._lib as L
    q = _Q(width)
    L.ensure_slots(bank.desc, layer, dist_dev, q0, width, record, q.ms, q.mk, q.nm, _stream())
    torch.cuda.synchronize()
    n = int(q.nm.item())
    return q.ms.cpu().numpy()[:n].tolist(), q.mk.cpu().numpy()[:n].tolist()


def _run_both(bank, st, layer, distinct, width, record, where):
    d = torch.from_numpy(np.ascontiguousarray(distinct.astype(np.int32))).cuda()
    splits = []
    for q0 in range(0, distinct.size, width):
        w = min(width, distinct.size - q0)
        gs, gk = _ensure_gpu(bank, layer, d, q0, w, record)
        rs, rk = ensure_slots(st, layer, distinct[q0:q0 + w], record)
        assert (gs, gk) == (rs, rk), f"{where} query at {q0}"
        _same_state(bank, st, f"{where} query at {q0}")
        splits.append(len(gs))
    return splits


def test_short_prefill_admission_split_and_state():
    row = [r for r in read_golden("lru_query_splits.txt") if r[0] == "short_prefill_96"][0]
    want = [int(v) for v in row[4:]]
    cfg = W.C2
    lg, _ = W.logits_with_chosen(cfg.seed, cfg.T, cfg.shape.E, cfg.shape.k, 160)
    ids, _ = route_topk_softmax(lg, cfg.shape.k)
    distinct, cnt, _ = dedup_sorted(ids.reshape(-1), cfg.shape.E)
    fill = W.bank_prefilled(cfg.seed, cfg.S, cfg.L, cfg.shape.E, 600, exclude_layer=0)
    bank = _bank(cfg.S, cfg.L, cfg.shape.E)
    bank.load_fill(fill)
    st = SlotBankState.from_fill(fill)
    _same_state(bank, st, "after fill")
    assert _run_both(bank, st, 0, distinct, cfg.W, False, "short prefill") == want
    assert np.all(bank.snapshot()["stats"] == 0)


def test_one_layer_cache_three_per_query():
    row = [r for r in read_golden("lru_query_splits.txt") if r[0] == "layer_view_s8"][0]
    want = [int(v) for v in row[4:]]
    fill = W.bank_prefilled(3, 8, 48, 8, 8, exclude_layer=0)
    bank = _bank(8, 48, 8)
    bank.load_fill(fill)
    st = SlotBankState.from_fill(fill)
    assert _run_both(bank, st, 0, np.arange(8, dtype=np.int32), 3, False, "s8") == want


def test_random_queries_with_evictions_and_stats():
    g = np.random.default_rng(21)
    S, NL, E = 64, 3, 40
    bank = _bank(S, NL, E)
    st = SlotBankState(S, NL, E)
    for i in range(300):
        layer = int(g.integers(0, NL))
        w = int(g.integers(1, 21))
        q = np.sort(g.choice(E, size=w, replace=False)).astype(np.int32)
        if g.random() < 0.2:
            q = np.concatenate([q, np.full(int(g.integers(1, 4)), E, np.int32)])  # sentinel tail
        _run_both(bank, st, layer, q, q.size, bool(g.integers(0, 2)), f"step {i}")


def test_decode_stream_zipf_against_oracle():
    cfg = W.C4
    S, NL, E, k = cfg.S, cfg.L, cfg.shape.E, cfg.shape.k
    steps = 12
    flush(f"decode zipf S={S} layers={NL} steps={steps}")
    bank = _bank(S, NL, E)
    st = SlotBankState(S, NL, E)
    misses = []
    for step in range(steps):
        for layer in range(NL):
            lg = W.zipf_gumbel_logits(cfg.seed, layer, step, cfg.T, E)
            ids, _ = route_topk_softmax(lg, k)
            distinct, cnt, _ = dedup_sorted(ids.reshape(-1), E)
            d = torch.from_numpy(distinct).cuda()
            gs, gk = _ensure_gpu(bank, layer, d, 0, distinct.size, True)
            rs, rk = ensure_slots(st, layer, distinct, True)
            assert (gs, gk) == (rs, rk), (step, layer)
            misses.append(len(gs))
    _same_state(bank, st, "end of decode")
    s = bank.snapshot()["stats"]
    assert s[1] > 0 and s[2] > 0, "the stream forces evictions"
    assert int(s[3]) == steps * NL


def test_capacity_error_is_sticky_and_partial():
    bank = _bank(4, 1, 16)
    st = SlotBankState(4, 1, 16)
    _run_both(bank, st, 0, np.arange(5, dtype=np.int32), 5, False, "overflow")
    assert bank.snapshot()["err"] == 1
    _run_both(bank, st, 0, np.array([9], np.int32), 1, True, "next call")
    assert bank.snapshot()["err"] == 1


def test_widest_query():
    S, E = 3000, 4096
    bank = _bank(S, 1, E)
    st = SlotBankState(S, 1, E)
    q = np.sort(np.random.default_rng(2).choice(E, 1024, replace=False)).astype(np.int32)
    _run_both(bank, st, 0, q, 1024, True, "w1024")
    q2 = np.sort(np.random.default_rng(3).choice(E, 1024, replace=False)).astype(np.int32)
    _run_both(bank, st, 0, q2, 1024, True, "w1024 b")


def test_copy_misses_bytes_equal_host_and_others_untouched():
    import slot_cache_routed_amd.layer as LY
    import slot_cache_routed_amd._lib as L
    S, NL, E = 40, 3, 24
    rec = 3 * 65536 + 4096            # a partial last chunk
    g = np.random.default_rng(5)
    pool = LY.HostPool(NL, E, rec, NL * E)
    for p in range(NL * E):
        pool.write_payload(p, g.integers(0, 256, size=rec, dtype=np.uint8))
    bank = LY.Bank(S, NL, E, 0, rec)
    bank.rows.copy_(torch.from_numpy(g.integers(0, 256, size=S * rec, dtype=np.uint8)).cuda())
    fill = W.bank_prefilled(7, S, NL, E, 30, exclude_layer=0)
    bank.load_fill(fill)
    before = bank.rows.clone()
    st = SlotBankState.from_fill(fill)
    distinct = np.sort(g.choice(E, 16, replace=False)).astype(np.int32)
    d = torch.from_numpy(distinct).cuda()
    admitted = []
    for q0 in range(0, 16, 6):
        w = min(6, 16 - q0)
        q = _Q(w)
        L.ensure_slots(bank.desc, 0, d, q0, w, 0, q.ms, q.mk, q.nm, _stream())
        L.copy_misses(bank.desc, pool.desc, q.ms, q.mk, q.nm, w, _stream())
        rs, rk = ensure_slots(st, 0, distinct[q0:q0 + w], False)
        admitted += list(zip(rs, rk))
    torch.cuda.synchronize()
    _same_state(bank, st, "after copies")
    assert len(admitted) == 16
    touched = set()
    for s, key in admitted:
        assert torch.equal(bank.slot_record(s).cpu(), pool.key_record(key)), (s, key)
        touched.add(s)
    for s in range(S):
        if s not in touched:
            assert torch.equal(bank.slot_record(s), before[s * rec:(s + 1) * rec]), s


def test_batched_admission_equals_query_by_query():
    """One launch for all queries of a chunk gives the per-query splits, bank
    state and output bits of the query-by-query admission."""
    import slot_cache_routed_amd.layer as LY
    import slot_cache_routed_amd._lib as L
    from helpers import ExpertSource, fill_pool
    cfg = W.C2
    E, k, H, I, S, NL, T = cfg.shape.E, cfg.shape.k, cfg.shape.H, cfg.shape.I, cfg.S, cfg.L, cfg.T
    lay = LY.record_layout(L.SCR_W_BF16, H, I)
    src = ExpertSource(cfg.seed, H, I, "bf16")
    pool = LY.HostPool(NL, E, lay.record_bytes, E, payload_of=lambda key: key % E)
    fill_pool(pool, src, lay, range(E))
    lg, _ = W.logits_with_chosen(cfg.seed, T, E, k, 160)
    xb = W.f32_to_bf16_bits(W.activations_normal(cfg.seed, T, H))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    sc = dev(np.ones(E, np.float32))
    fill = W.bank_prefilled(cfg.seed, S, NL, E, 600, exclude_layer=0)
    res = []
    for batched in (False, True):
        bank = LY.Bank(S, NL, E, L.SCR_W_BF16, lay.record_bytes)
        bank.load_fill(fill)
        d = LY.demand_layer(bank, pool, 0, dev(lg), dev(xb.view(np.int16)), sc, width=128, shape=(k, H, I),
                            batched=batched)
        torch.cuda.synchronize()
        res.append((d["n_miss"].cpu().numpy().tolist(), bank.snapshot(), d["y"].clone(), bank.rows.clone()))
    assert res[0][0] == res[1][0] == [128, 32, 0, 0]
    for key in ("slot_key", "key_to_slot", "slot_stamp", "stats", "clock"):
        assert np.array_equal(np.asarray(res[0][1][key]), np.asarray(res[1][1][key])), key
    assert torch.equal(res[0][2], res[1][2]) and torch.equal(res[0][3], res[1][3])


def test_batched_admission_supersedes_re_evicted_entries():
    """A bank too small for the chunk (10 experts, 6 slots, queries of 4): later
    queries take the first query's slots again; the list marks those entries
    superseded and every slot ends with its final owner's record."""
    import slot_cache_routed_amd.layer as LY
    import slot_cache_routed_amd._lib as L
    S, NL, E, rec = 6, 1, 16, 4096
    g = np.random.default_rng(4)
    pool = LY.HostPool(NL, E, rec, E)
    for p in range(E):
        pool.write_payload(p, g.integers(0, 256, size=rec, dtype=np.uint8))
    bank = LY.Bank(S, NL, E, 0, rec)
    distinct = torch.arange(10, dtype=torch.int32, device="cuda")      # 10 experts, 6 slots, queries of 4
    ms = torch.full((10,), -9, dtype=torch.int32, device="cuda")
    mk = torch.full((10,), -9, dtype=torch.int32, device="cuda")
    nm = torch.zeros(3, dtype=torch.int32, device="cuda")
    nt = torch.zeros(1, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    L.ensure_slots_batched(bank.desc, 0, distinct, 10, 4, 0, ms, mk, nm, nt, s)
    L.copy_misses(bank.desc, pool.desc, ms, mk, nt, 10, s)
    torch.cuda.synchronize()
    st = SlotBankState(S, NL, E)
    splits = []
    for q0 in range(0, 10, 4):
        splits.append(len(ensure_slots(st, 0, np.arange(q0, min(10, q0 + 4), dtype=np.int32), False)[0]))
    snap = bank.snapshot()
    for key in ("slot_key", "key_to_slot", "slot_stamp", "clock"):
        assert np.array_equal(np.asarray(snap[key]), np.asarray(getattr(st, key))), key
    assert nm.cpu().numpy().tolist() == splits == [4, 4, 2] and snap["err"] == st.err == 0
    slots = ms.cpu().numpy()[:int(nt.item())]
    assert (slots < 0).sum() == 4, "the first query's four admissions were taken again"
    for sl in range(S):
        key = int(snap["slot_key"][sl])
        assert torch.equal(bank.slot_record(sl).cpu(), pool.key_record(key))


def test_batched_admission_on_a_bank_past_the_prefetch_size():
    """The batched planner reads every query entry's slot up front only for
    banks of at most 65536 slots; a bank of 70000 slots takes the per-query
    lookups.  Three chunks (300 distinct experts in queries of 128, then
    overlapping ones) against the oracle, bank state bit-exact after each."""
    import slot_cache_routed_amd._lib as L
    S, NL, E = 70000, 2, 512
    bank = _bank(S, NL, E)
    st = SlotBankState(S, NL, E)
    g = np.random.default_rng(70000)
    s = _stream()
    for chunk in range(3):
        layer = chunk % NL
        distinct = np.sort(g.choice(E, size=300, replace=False)).astype(np.int32)
        flush(f"batched past prefetch: chunk {chunk}, layer {layer}")
        d = torch.from_numpy(distinct).cuda()
        ms = torch.full((300,), -9, dtype=torch.int32, device="cuda")
        mk = torch.full((300,), -9, dtype=torch.int32, device="cuda")
        nm = torch.zeros(3, dtype=torch.int32, device="cuda")
        nt = torch.zeros(1, dtype=torch.int32, device="cuda")
        L.ensure_slots_batched(bank.desc, layer, d, 300, 128, 1, ms, mk, nm, nt, s)
        torch.cuda.synchronize()
        splits, slots, keys = [], [], []
        for q0 in range(0, 300, 128):
            rs, rk = ensure_slots(st, layer, distinct[q0:q0 + 128], True)
            splits.append(len(rs))
            slots += rs
            keys += rk
        assert nm.cpu().numpy().tolist() == splits
        n = int(nt.item())
        assert ms.cpu().numpy()[:n].tolist() == slots and mk.cpu().numpy()[:n].tolist() == keys
        _same_state(bank, st, f"chunk {chunk}")
