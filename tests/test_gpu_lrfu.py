"""GPU parity of the scored (LRFU) eviction: the bank state, including every
slot's fixed-point value, bit-exact against the oracle after every query of
a decode-like stream whose chunks span several queries (the pin), the batched
and one-launch planners equal to query-by-query admission, and the hand-worked
two-slot example through the C ABI."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from conftest import read_golden
from helpers import ExpertSource, fill_pool, flush
from oracle import SlotBankState, dedup_sorted, ensure_slots, route_topk_softmax
from oracle.lru import POLICY_LRFU, POLICY_LRU

pytestmark = pytest.mark.gpu

STATE = ("slot_key", "key_to_slot", "slot_stamp", "stats", "decode_freq", "slot_crf")


def _decay(h):
    return math.floor(2 ** 32 * 2 ** (-1.0 / h))


def _state(st):
    return {"slot_key": st.slot_key, "key_to_slot": st.key_to_slot, "slot_stamp": st.slot_stamp,
            "stats": st.stats, "decode_freq": st.decode_freq, "slot_crf": st.slot_crf}


def _setup(T=4, E=64, k=6, H=128, I=128, NL=4, seed=61):
    import slot_cache_routed_amd._lib as L
    import slot_cache_routed_amd.layer as LY
    lay = LY.record_layout(L.SCR_W_BF16, H, I)
    src = ExpertSource(seed, H, I, "bf16")
    pool = LY.HostPool(NL, E, lay.record_bytes, E, payload_of=lambda key: key % E)
    fill_pool(pool, src, lay, range(E))
    return L, LY, lay, pool


@pytest.mark.parametrize("h", [2, 8, 64])
def test_lrfu_stream_state_bit_exact_after_every_layer_step(h):
    L, LY, lay, pool = _setup()
    T, E, k, H, I, NL, S, W_ = 4, 64, 6, 128, 128, 4, 100, 8
    D = _decay(h)
    bank = LY.Bank(S, NL, E, L.SCR_W_BF16, lay.record_bytes, policy=L.SCR_POLICY_LRFU, lrfu_decay=D)
    st = SlotBankState(S, NL, E)
    st.policy, st.decay_q32 = POLICY_LRFU, D
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    sc = dev(np.ones(E, np.float32))
    buf = LY.LayerBuffers(T, E, k, H, I, S, L.SCR_W_BF16, width=W_)
    for step in range(8):
        for layer in range(NL):
            lg = W.zipf_gumbel_logits(61, layer, step, T, E)
            xb = W.f32_to_bf16_bits(W.decode_activations(61, layer, step, T, H))
            LY.demand_layer(bank, pool, layer, dev(lg), dev(xb.view(np.int16)), sc, width=W_, record_stats=True,
                            buf=buf, shape=(k, H, I))
            ids, _ = route_topk_softmax(lg, k)
            distinct, nd, _ = dedup_sorted(ids.reshape(-1), E)
            for q0 in range(0, len(distinct), W_):
                ensure_slots(st, layer, distinct[q0:q0 + W_], True, chunk_first=(q0 == 0))
            snap = bank.snapshot()
            for key in STATE:
                assert np.array_equal(np.asarray(snap[key]), np.asarray(_state(st)[key])), (step, layer, key)
            assert snap["clock"] == st.clock and snap["err"] == st.err == 0
    hits, misses, ev, _ = [int(v) for v in st.stats]
    flush(f"lrfu h={h}: hits {hits} misses {misses} evictions {ev}")
    assert ev > 0 and hits > 0


@pytest.mark.parametrize("planner", ["batched", "plan_chunk"])
def test_lrfu_batched_and_one_launch_planners_equal_query_by_query(planner):
    L, LY, lay, pool = _setup()
    T, E, k, H, I, NL, S, W_ = 4, 64, 6, 128, 128, 4, 100, 8
    D = _decay(8)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    sc = dev(np.ones(E, np.float32))
    banks = [LY.Bank(S, NL, E, L.SCR_W_BF16, lay.record_bytes, policy=L.SCR_POLICY_LRFU, lrfu_decay=D)
             for _ in range(2)]
    bufs = [LY.LayerBuffers(T, E, k, H, I, S, L.SCR_W_BF16, width=W_) for _ in range(2)]
    for step in range(6):
        for layer in range(NL):
            lg = dev(W.zipf_gumbel_logits(62, layer, step, T, E))
            xb = dev(W.f32_to_bf16_bits(W.decode_activations(62, layer, step, T, H)).view(np.int16))
            LY.demand_layer(banks[0], pool, layer, lg, xb, sc, width=W_, record_stats=True, buf=bufs[0],
                            shape=(k, H, I))
            LY.demand_layer(banks[1], pool, layer, lg, xb, sc, width=W_, record_stats=True, buf=bufs[1],
                            shape=(k, H, I), batched=planner == "batched", fused=planner == "plan_chunk")
            a, b = banks[0].snapshot(), banks[1].snapshot()
            for key in STATE + ("clock",):
                assert np.array_equal(np.asarray(a[key]), np.asarray(b[key])), (step, layer, key)
            assert torch.equal(bufs[0]["y"], bufs[1]["y"])
            assert torch.equal(banks[0].rows, banks[1].rows)


def test_lrfu_worked_example_through_the_abi():
    L, LY, lay, pool = _setup(E=4, NL=1)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    s = torch.cuda.current_stream().cuda_stream
    for policy, seq, victim, evicted in read_golden("lrfu_worked_example.txt"):
        pol = L.SCR_POLICY_LRFU if policy == "lrfu" else L.SCR_POLICY_LRU
        bank = LY.Bank(2, 1, 4, L.SCR_W_BF16, lay.record_bytes, policy=pol, lrfu_decay=_decay(2))
        ms, mk, nm = (torch.zeros(1, dtype=torch.int32, device="cuda") for _ in range(3))
        experts = [int(x) for x in seq.split(",")]
        for e in experts[:-1]:
            L.ensure_slots(bank.desc, 0, dev([e]), 0, 1, 0, ms, mk, nm, s)
        before = bank.snapshot()
        L.ensure_slots(bank.desc, 0, dev([experts[-1]]), 0, 1, 0, ms, mk, nm, s)
        torch.cuda.synchronize()
        assert int(nm.item()) == 1 and int(ms.item()) == int(victim) and int(mk.item()) == experts[-1]
        assert before["slot_key"][int(victim)] == int(evicted)


def test_lrfu_capacity_overflow_within_a_pinned_chunk():
    # a chunk of three queries needing more slots than the bank has: the pin
    # keeps its earlier admissions, so the last query's surplus misses set the
    # capacity bit instead of evicting them (oracle and device alike)
    L, LY, lay, pool = _setup(E=64, NL=1)
    S, W_ = 10, 6
    D = _decay(8)
    bank = LY.Bank(S, 1, 64, L.SCR_W_BF16, lay.record_bytes, policy=L.SCR_POLICY_LRFU, lrfu_decay=D)
    st = SlotBankState(S, 1, 64)
    st.policy, st.decay_q32 = POLICY_LRFU, D
    s = torch.cuda.current_stream().cuda_stream
    distinct = np.arange(3, 3 + 18, dtype=np.int32)           # 18 distinct experts, 3 queries of 6
    dev_d = torch.from_numpy(distinct).cuda()
    ms = torch.full((W_,), -1, dtype=torch.int32, device="cuda")
    mk = torch.full((W_,), -1, dtype=torch.int32, device="cuda")
    nm = torch.zeros(1, dtype=torch.int32, device="cuda")
    for q0 in range(0, 18, W_):
        L.ensure_slots(bank.desc, 0, dev_d, q0, W_, 1, ms, mk, nm, s)
        rs, _ = ensure_slots(st, 0, distinct[q0:q0 + W_], True, chunk_first=(q0 == 0))
        torch.cuda.synchronize()
        assert int(nm.item()) == len(rs) and ms.cpu().numpy()[:len(rs)].tolist() == rs, q0
    snap = bank.snapshot()
    for key in STATE:
        assert np.array_equal(np.asarray(snap[key]), np.asarray(_state(st)[key])), key
    assert snap["err"] == st.err == 1
    assert sorted(int(k) for k in snap["slot_key"]) == list(range(3, 13))   # the first ten admissions stay


def test_lrfu_decode_stream_at_full_planner_scale():
    """The decode stream's planner scale (48 layers x 512 experts, a 1650-slot
    bank, 4-token steps, top-10 Zipf(1.1) routing) under LRFU with a half-life
    of 16 queries: the bank state, every slot's value included, bit-exact
    against the oracle after every layer-step of 4 steps.  Records are small
    (hidden 128, intermediate 128): the GEMM sizes do not enter the planner."""
    cfg = W.C4
    E, k, S, NL, T = cfg.shape.E, cfg.shape.k, cfg.S, cfg.L, cfg.T
    H = I = 128
    L, LY, lay, pool = _setup(T=T, E=E, k=k, H=H, I=I, NL=NL, seed=cfg.seed)
    D = _decay(16)
    bank = LY.Bank(S, NL, E, L.SCR_W_BF16, lay.record_bytes, policy=L.SCR_POLICY_LRFU, lrfu_decay=D)
    st = SlotBankState(S, NL, E)
    st.policy, st.decay_q32 = POLICY_LRFU, D
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    sc = dev(np.ones(E, np.float32))
    buf = LY.LayerBuffers(T, E, k, H, I, S, L.SCR_W_BF16, width=128)
    for step in range(4):
        flush(f"LRFU decode at full planner scale: step {step}")
        for layer in range(NL):
            lg = W.zipf_gumbel_logits(cfg.seed, layer, step, T, E)
            xb = W.f32_to_bf16_bits(W.decode_activations(cfg.seed, layer, step, T, H))
            LY.demand_layer(bank, pool, layer, dev(lg), dev(xb.view(np.int16)), sc, width=128, record_stats=True,
                            buf=buf, shape=(k, H, I))
            ids, _ = route_topk_softmax(lg, k)
            distinct, _, _ = dedup_sorted(ids.reshape(-1), E)
            ensure_slots(st, layer, distinct, True)
            torch.cuda.synchronize()
            snap = bank.snapshot()
            for key in STATE:
                assert np.array_equal(np.asarray(snap[key]), np.asarray(_state(st)[key])), (step, layer, key)
    hits, misses, evictions, queries = [int(v) for v in bank.snapshot()["stats"]]
    flush(f"LRFU decode at full planner scale: hits {hits} misses {misses} evictions {evictions}")
    assert queries == 4 * NL and evictions > 0
