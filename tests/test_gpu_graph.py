"""The demand step holds no host sync, so it can be captured as a HIP graph:
replays (with eager work and synchronisations between them) give the eager
step's bits, and the bank keeps evolving as in eager execution."""
import numpy as np
import pytest
import torch

import workloads as W
from helpers import ExpertSource, fill_pool

pytestmark = pytest.mark.gpu


def test_captured_demand_step_replays_bitwise():
    import slot_cache_routed_amd._lib as L
    import slot_cache_routed_amd.layer as LY
    T, E, k, H, I, S, NL = 48, 64, 6, 512, 256, 96, 4
    lay = LY.record_layout(L.SCR_W_BF16, H, I)
    src = ExpertSource(31, H, I, "bf16")
    pool = LY.HostPool(NL, E, lay.record_bytes, E, payload_of=lambda key: key % E)
    fill_pool(pool, src, lay, range(E))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    sc = dev(np.ones(E, np.float32))
    logits = [dev(W.logits_normal(31, l, T, E)) for l in range(NL)]
    x = dev(W.f32_to_bf16_bits(W.activations_normal(31, T, H)).view(np.int16))

    def run(bank, buf, layer):
        LY.demand_layer(bank, pool, layer, logits[layer], x, sc, width=32, record_stats=True, buf=buf,
                        shape=(k, H, I))

    # eager reference: layers 0..3 then 0 again
    bank_e = LY.Bank(S, NL, E, L.SCR_W_BF16, lay.record_bytes)
    buf_e = LY.LayerBuffers(T, E, k, H, I, S, L.SCR_W_BF16, width=32)
    ref = []
    for layer in (0, 1, 2, 3, 0):
        run(bank_e, buf_e, layer)
        ref.append(buf_e["y"].clone())
    torch.cuda.synchronize()

    # graph: one captured step per layer, replayed in the same order
    bank_g = LY.Bank(S, NL, E, L.SCR_W_BF16, lay.record_bytes)
    bufs = [LY.LayerBuffers(T, E, k, H, I, S, L.SCR_W_BF16, width=32) for _ in range(NL)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graphs = []
    with torch.cuda.stream(side):
        for layer in range(NL):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                run(bank_g, bufs[layer], layer)
            graphs.append(g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    # capture enqueued nothing: the bank is still empty
    assert int(bank_g.clock.item()) == 0
    out = []
    for i, layer in enumerate((0, 1, 2, 3, 0)):
        graphs[layer].replay()
        torch.cuda.synchronize()
        out.append(bufs[layer]["y"].clone())
        _ = (x.float() * 2).sum().item()      # eager work between replays
    for a, b in zip(ref, out):
        assert torch.equal(a, b)
    se, sg = bank_e.snapshot(), bank_g.snapshot()
    for key in ("slot_key", "key_to_slot", "slot_stamp", "stats", "decode_freq", "clock"):
        assert np.array_equal(np.asarray(se[key]), np.asarray(sg[key])), key


@pytest.mark.parametrize("fused", [False, True])
def test_captured_decode_step_of_all_layers_replays_bitwise(fused):
    """A whole decode step (every layer's route, planning, miss copies and
    GEMMs) in one graph, replayed over several steps with new inputs written
    into its static tensors: the same outputs and bank as eager steps, with
    hits and evictions (a bank smaller than the layers' experts)."""
    import slot_cache_routed_amd._lib as L
    import slot_cache_routed_amd.layer as LY
    T, E, k, H, I, S, NL, steps = 4, 64, 6, 256, 128, 96, 5, 5
    lay = LY.record_layout(L.SCR_W_BF16, H, I)
    src = ExpertSource(57, H, I, "bf16")
    pool = LY.HostPool(NL, E, lay.record_bytes, E, payload_of=lambda key: key % E)
    fill_pool(pool, src, lay, range(E))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    sc = dev(np.ones(E, np.float32))
    logits = [[dev(W.zipf_gumbel_logits(57, l, st, T, E)) for l in range(NL)] for st in range(steps)]
    xs = [[dev(W.f32_to_bf16_bits(W.decode_activations(57, l, st, T, H)).view(np.int16)) for l in range(NL)]
          for st in range(steps)]

    bank_e = LY.Bank(S, NL, E, L.SCR_W_BF16, lay.record_bytes)
    bufs_e = [LY.LayerBuffers(T, E, k, H, I, S, L.SCR_W_BF16, width=16, y_dtype=L.SCR_Y_BF16) for _ in range(NL)]
    ref = []
    for st in range(steps):
        for l in range(NL):
            LY.demand_layer(bank_e, pool, l, logits[st][l], xs[st][l], sc, width=16, record_stats=True,
                            buf=bufs_e[l], shape=(k, H, I), batched=True, fused=fused)
            ref.append(bufs_e[l]["y"].clone())
    torch.cuda.synchronize()

    bank_g = LY.Bank(S, NL, E, L.SCR_W_BF16, lay.record_bytes)
    step = LY.DecodeStepGraph(bank_g, pool, range(NL), T, E, (k, H, I), sc, width=16, record_stats=True,
                              y_dtype=L.SCR_Y_BF16, fused=fused)
    torch.cuda.synchronize()
    assert int(bank_g.clock.item()) == 0            # capture enqueued nothing
    out = []
    for st in range(steps):
        for l in range(NL):
            step.logits[l].copy_(logits[st][l])
            step.x[l].copy_(xs[st][l])
        step.replay()
        torch.cuda.synchronize()
        out.extend(step.bufs[l]["y"].clone() for l in range(NL))
        _ = (xs[st][0].float() * 3).sum().item()    # eager work between replays
    for i, (a, b) in enumerate(zip(ref, out)):
        assert torch.equal(a, b), f"step {i // NL} layer {i % NL}"
    se, sg = bank_e.snapshot(), bank_g.snapshot()
    for key in ("slot_key", "key_to_slot", "slot_stamp", "stats", "decode_freq", "clock", "err"):
        assert np.array_equal(np.asarray(se[key]), np.asarray(sg[key])), key
    hits, misses, evictions, queries = [int(v) for v in sg["stats"]]
    assert evictions > 0 and hits > 0 and queries == steps * NL * step.bufs[0].n_queries
