"""GPU parity of the decode stream: 48 layers x 512 experts sharing a
1650-slot bank, 4-token steps with Zipf(1.1)-skewed routing, decode
statistics on, from an empty bank, 32 steps.  Every layer-step runs the whole
slot path through the C ABI (route, dedup, one LRU query, miss copy, align
over the slots, grouped GEMM; even steps plan each layer in one launch, odd
steps with the separate calls); the bank state and statistics are compared
bit for bit with the oracle after every layer-step, and the outputs of two
layers of every step against the oracle within tolerance."""
import numpy as np
import pytest
import torch

import workloads as W
from concurrent.futures import ThreadPoolExecutor

from helpers import N_THREADS, ExpertSource, fill_pool, flush, rel_max_err
from oracle import SlotBankState, dedup_sorted, ensure_slots, moe_layer, route_topk_softmax
from oracle.mlp import bf16_bits_to_f64

pytestmark = pytest.mark.gpu

N_PAYLOADS = 512     # keys (layer, e) share records e: bounded pinned memory


def test_decode_stream_state_and_outputs():
    import slot_cache_routed_amd._lib as L
    import slot_cache_routed_amd.layer as LY
    cfg = W.C4
    E, k, H, I, S, NL, T = cfg.shape.E, cfg.shape.k, cfg.shape.H, cfg.shape.I, cfg.S, cfg.L, cfg.T
    steps = 32
    lay = LY.record_layout(L.SCR_W_BF16, H, I)
    src = ExpertSource(cfg.seed, H, I, "bf16")
    flush(f"decode: {NL} layers x {E} experts, S={S}, {steps} steps of {T} tokens")
    pool = LY.HostPool(NL, E, lay.record_bytes, N_PAYLOADS, payload_of=lambda key: key % N_PAYLOADS)
    fill_pool(pool, src, lay, range(N_PAYLOADS))
    bank = LY.Bank(S, NL, E, L.SCR_W_BF16, lay.record_bytes)
    st = SlotBankState(S, NL, E)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    sc = dev(np.ones(E, np.float32))
    buf = LY.LayerBuffers(T, E, k, H, I, S, L.SCR_W_BF16, width=128)
    checked = 0
    for step in range(steps):
        for layer in range(NL):
            lg = W.zipf_gumbel_logits(cfg.seed, layer, step, T, E)
            xb = W.f32_to_bf16_bits(W.decode_activations(cfg.seed, layer, step, T, H))
            LY.demand_layer(bank, pool, layer, dev(lg), dev(xb.view(np.int16)), sc, width=128, record_stats=True,
                            buf=buf, shape=(k, H, I), fused=step % 2 == 0)
            ids, w = route_topk_softmax(lg, k)
            distinct, _, _ = dedup_sorted(ids.reshape(-1), E)
            rs, rk = ensure_slots(st, layer, distinct, True)
            torch.cuda.synchronize()
            assert int(buf["n_miss"][0].item()) == len(rs), (step, layer)
            snap = bank.snapshot()
            for key in ("slot_key", "key_to_slot", "slot_stamp", "stats", "decode_freq"):
                assert np.array_equal(snap[key], getattr(st, key)), (step, layer, key)
            assert snap["err"] == 0, (step, layer)
            if layer in (step % NL, (7 * step + 3) % NL):
                y = buf["y"].cpu().numpy()
                pays = sorted({int(e) % N_PAYLOADS for e in ids.reshape(-1)})
                with ThreadPoolExecutor(N_THREADS) as ex:       # the routed experts' fp64 weights
                    wts = dict(zip(pays, ex.map(src.f64, pays)))
                y_ref = moe_layer(bf16_bits_to_f64(xb), ids, w, lambda e: wts[e % N_PAYLOADS])
                assert rel_max_err(y, y_ref) <= 2e-2, (step, layer)
                checked += 1
    snap = bank.snapshot()
    for key in ("slot_key", "key_to_slot", "slot_stamp", "stats", "decode_freq"):
        assert np.array_equal(snap[key], getattr(st, key)), key
    assert snap["clock"] == st.clock == steps * NL and snap["err"] == 0
    hits, misses, evictions, queries = [int(v) for v in snap["stats"]]
    flush(f"decode: hits {hits} misses {misses} evictions {evictions} queries {queries}; outputs checked {checked}")
    assert evictions > 0 and queries == steps * NL and checked >= steps
