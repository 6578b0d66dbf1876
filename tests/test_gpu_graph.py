"""The demand step holds no host sync, so it can be captured as a HIP graph:
replays (with eager work and synchronisations between them) give the eager
step's bits, and the bank keeps evolving as in eager execution."""
import numpy as np
import pytest
import torch

import workloads as W
from helpers import ExpertSource, fill_pool, flush

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


def test_short_prefill_96_step_as_the_bench_times_it():
    """The 96-token chunk over the 1100-slot bank exactly as the benchmark runs
    it: route, the one-launch planner, the miss copy, the grouped GEMMs and a
    bf16 combine, then the warm step captured once and replayed.  The cold step
    admits 128 + 32 experts and matches the oracle; every replay equals the
    eager warm step and the whole-layer stream bit for bit."""
    import slot_cache_routed_amd._lib as L
    import slot_cache_routed_amd.layer as LY
    from oracle import moe_layer, route_topk_softmax
    from oracle.mlp import bf16_bits_to_f64
    from helpers import rel_max_err
    cfg = W.C2
    T, E, k, H, I, S, NL, Wd = cfg.T, cfg.shape.E, cfg.shape.k, cfg.shape.H, cfg.shape.I, cfg.S, cfg.L, cfg.W
    lay = LY.record_layout(L.SCR_W_BF16, H, I)
    src = ExpertSource(cfg.seed, H, I, "bf16")
    pool = LY.HostPool(NL, E, lay.record_bytes, E, payload_of=lambda key: key % E)
    fill_pool(pool, src, lay, range(E))
    lg, _ = W.logits_with_chosen(cfg.seed, T, E, k, 160)
    xb = W.f32_to_bf16_bits(W.activations_normal(cfg.seed, T, H))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    logits, x, sc = dev(lg), dev(xb.view(np.int16)), dev(np.ones(E, np.float32))
    bank = LY.Bank(S, NL, E, L.SCR_W_BF16, lay.record_bytes)
    bank.load_fill(W.bank_prefilled(cfg.seed, S, NL, E, 600, exclude_layer=0))
    buf = LY.LayerBuffers(T, E, k, H, I, S, L.SCR_W_BF16, width=Wd, y_dtype=L.SCR_Y_BF16)
    view = LY.make_view(0, E, k, H, I, L.SCR_W_BF16, S, bank.row_table, sc)

    def step(s):
        L.route(logits, T, E, k, buf["topk_ids"], buf["topk_w"], s)
        assert L.plan_chunk(bank.desc, 0, buf["topk_ids"], buf.R, buf["distinct"], buf["n_distinct"], Wd, False,
                            buf["miss_slot"], buf["miss_key"], buf["n_miss"], buf["n_total"], buf.cfg.block_m,
                            buf["sorted_routes"], buf["block_bucket"], buf["n_post_pad"], buf["active_buckets"],
                            buf["active_block_begin"], buf["n_active"], s)
        L.copy_misses(bank.desc, pool.desc, buf["miss_slot"], buf["miss_key"], buf["n_total"], buf.lmax, s)
        LY.forward(buf, view, x, stream=torch.cuda.current_stream())

    flush("96-token step: cold")
    step(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert buf["n_miss"].cpu().numpy().tolist() == [128, 32, 0, 0]
    y_cold = buf["y"].clone()
    # the same plan through the fp32-output mode: within the bf16 tolerance of
    # the oracle, and the benchmarked bf16 output is exactly its rounding
    buf32 = LY.LayerBuffers(T, E, k, H, I, S, L.SCR_W_BF16, width=Wd, y_dtype=L.SCR_Y_F32)
    for key in ("topk_w", "sorted_routes", "active_buckets", "active_block_begin", "n_active"):
        buf32[key].copy_(buf[key])
    LY.forward(buf32, view, x)
    torch.cuda.synchronize()
    y32 = buf32["y"].clone()
    assert torch.equal(y_cold, y32.to(torch.bfloat16))
    ids, w = route_topk_softmax(lg, k)
    y_ref = moe_layer(bf16_bits_to_f64(xb), ids, w, src.f64)
    err = rel_max_err(y32.cpu().numpy(), y_ref)
    flush(f"96-token step: rel max err {err:.3e} (fp32 output of the same plan)")
    assert err <= 2e-2
    flush("96-token step: warm, eager then captured")
    step(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    y_warm = buf["y"].clone()
    assert torch.equal(y_warm, y_cold) and buf["n_miss"].cpu().numpy().sum() == 0
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            step(side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    # every launch of the step is in the graph: the route's and the planner's
    # outputs are cleared before each replay and come back, and the bank's
    # clock advances by one eager step's queries per replay
    plan_keys = ("topk_ids", "topk_w", "sorted_routes", "n_post_pad", "active_buckets", "active_block_begin",
                 "n_active")

    def plan_outputs():     # the defined parts of the route's and the planner's outputs
        n, npp = int(buf["n_active"][0]), int(buf["n_post_pad"][0])
        return [buf["topk_ids"].clone(), buf["topk_w"].clone(), buf["n_active"].clone(), buf["n_post_pad"].clone(),
                buf["active_buckets"][:n].clone(), buf["active_block_begin"][:n + 1].clone(),
                buf["sorted_routes"][:npp].clone()]

    plan_warm = plan_outputs()
    clock0 = bank.snapshot()["clock"]
    step(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    per_step = bank.snapshot()["clock"] - clock0
    assert per_step > 0
    for rep in range(3):
        buf["y"].zero_()
        for key in plan_keys:
            buf[key].fill_(-3)
        clock0 = bank.snapshot()["clock"]
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(buf["y"], y_warm)
        for i, (a, b) in enumerate(zip(plan_outputs(), plan_warm)):
            assert torch.equal(a, b), (rep, i)
        assert bank.snapshot()["clock"] - clock0 == per_step, rep
        _ = (x.float() * 2).sum().item()      # eager work between replays
    lb = LY.LayerStreamBuffer(E, lay.record_bytes)
    st = LY.stream_layer(pool, 0, logits, x, sc, lb, L.SCR_W_BF16, y_dtype=L.SCR_Y_BF16, shape=(k, H, I))
    torch.cuda.synchronize()
    assert torch.equal(st["y"], y_warm), "slot path equals the whole-layer path bit for bit"


@pytest.mark.parametrize("wd,T,E,k,H,I", [
    ("nvfp4", 4096, 512, 10, 2048, 512),    # the long-chunk NVFP4 layer: fp16 x copy, wide kernels
    ("mxfp4_a8", 1024, 64, 4, 2048, 512),   # W4A8: x quantised, fp8 x fp4 kernels
    ("bf16", 2048, 8, 2, 1024, 512),        # few experts: pass slices, split N chunks
])
def test_captured_long_chunk_forward_replays_bitwise(wd, T, E, k, H, I):
    """Route, align and the grouped GEMM of a long chunk over a resident layer,
    captured once and replayed three times (output overwritten with NaN and
    eager work between replays): every replay gives the eager bits."""
    import slot_cache_routed_amd._lib as L
    import slot_cache_routed_amd.layer as LY
    from helpers import wdtype_code
    code = wdtype_code(wd)
    lay = LY.record_layout(code, H, I)
    P = 16
    src = ExpertSource(41, H, I, wd)
    pool = LY.HostPool(1, E, lay.record_bytes, P, payload_of=lambda key: key % P)
    fill_pool(pool, src, lay, range(P))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    g = np.random.default_rng(41)
    sc = dev((0.5 + g.random(E)).astype(np.float32))
    sc2 = dev((0.25 + g.random(E)).astype(np.float32))
    lg = dev(W.logits_normal(41, 0, T, E))
    x = dev(W.f32_to_bf16_bits(W.activations_normal(41, T, H)).view(np.int16))
    lb = LY.LayerStreamBuffer(E, lay.record_bytes)
    kw = dict(shape=(k, H, I), down_input_scale=sc2)
    eager = LY.stream_layer(pool, 0, lg, x, sc, lb, code, **kw)   # also copies the layer in
    torch.cuda.synchronize()
    ref = eager["y"].clone()
    buf = LY.LayerBuffers(T, E, k, H, I, E, code)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            LY.stream_layer(pool, 0, lg, x, sc, lb, code, buf=buf, copy=False, **kw)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    flush(f"graph {wd} {T}x{E} k={k} H={H} I={I}: m_chunk {buf.cfg_used.m_chunk}")
    for rep in range(3):
        buf["y"].fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(buf["y"], ref), f"replay {rep}"
        _ = (x.float() * 2).sum().item()      # eager work between replays
