"""GPU parity of prefill staging: staged layers equal the whole-layer stream
bit for bit, resident bank rows stay untouched, every staged row equals its
host record, and every output element matches the oracle (NVFP4)."""
import numpy as np
import pytest
import torch

import workloads as W
from helpers import ExpertSource, fill_pool, flush, rel_max_err
from oracle import moe_layer, route_topk_softmax
from oracle.mlp import bf16_bits_to_f64

pytestmark = pytest.mark.gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _staging_case(T, n_layers, E, k, H, I, n_res, seed, S):
    import slot_cache_routed_amd._lib as L
    import slot_cache_routed_amd.layer as LY
    lay = LY.record_layout(L.SCR_W_NVFP4, H, I)
    src = ExpertSource(seed, H, I, "nvfp4")
    flush(f"staging case T={T} layers={n_layers} E={E} H={H} I={I} resident={n_res}")
    pool = LY.HostPool(n_layers, E, lay.record_bytes, n_layers * E)
    fill_pool(pool, src, lay, range(n_layers * E))
    bank = LY.Bank(S, n_layers, E, L.SCR_W_NVFP4, lay.record_bytes)
    # make each layer's resident set resident through the library's own admission
    s = torch.cuda.current_stream().cuda_stream
    for layer in range(n_layers if n_res else 0):
        res = W.resident_experts(seed, layer, E, n_res)
        d = _dev(res)
        ms = torch.zeros(n_res, dtype=torch.int32, device="cuda")
        mk = torch.zeros(n_res, dtype=torch.int32, device="cuda")
        nm = torch.zeros(1, dtype=torch.int32, device="cuda")
        L.ensure_slots(bank.desc, layer, d, 0, n_res, 0, ms, mk, nm, s)
        L.copy_misses(bank.desc, pool.desc, ms, mk, nm, n_res, s)
    torch.cuda.synchronize()
    return L, LY, lay, src, pool, bank


@pytest.mark.parametrize("T,n_layers,E,k,H,I,n_res,S", [
    (256, 3, 64, 6, 512, 256, 24, 100),
    (96, 2, 16, 4, 256, 128, 0, 40),      # nothing resident: every expert staged
    (96, 3, 16, 4, 256, 128, 16, 48),     # everything resident: nothing staged
    (4096, 2, 512, 10, 2048, 512, 193, 1650),
])
def test_staged_layers_equal_stream_and_oracle(T, n_layers, E, k, H, I, n_res, S):
    seed = 5
    L, LY, lay, src, pool, bank = _staging_case(T, n_layers, E, k, H, I, n_res, seed, S)
    rows_before = bank.rows.clone()
    sp = LY.StagedPrefill(bank, pool)
    n_runs = sp.plan(0, n_layers)
    for layer in range(n_layers):
        assert sp.staged_bytes(layer) == (E - n_res) * lay.record_bytes
    logits = [_dev(W.logits_normal(seed, layer, T, E)) for layer in range(n_layers)]
    xb = W.f32_to_bf16_bits(W.activations_normal(seed, T, H))
    x = _dev(xb.view(np.int16))
    sc = _dev(np.ones(E, np.float32))
    bufs = [LY.LayerBuffers(T, E, k, H, I, E, L.SCR_W_NVFP4) for _ in range(n_layers)]
    sp.run(list(range(n_layers)), logits, x, sc, bufs)
    torch.cuda.synchronize()
    assert torch.equal(bank.rows, rows_before), "resident rows untouched"
    # the last two staged layers (one per staging buffer): every non-resident
    # row equals its host record
    snap = bank.snapshot()
    n_checked = 0
    for layer in range(max(0, n_layers - 2), n_layers):
        staged = sp.staging[layer % 2].cpu().view(E, lay.record_bytes)
        for e in range(E):
            if snap["key_to_slot"][layer * E + e] < 0:
                assert torch.equal(staged[e], pool.key_record(layer * E + e)), (layer, e)
                n_checked += 1
    assert n_checked == min(2, n_layers) * (E - n_res)
    # whole-layer stream partner, same kernel and tiles
    lb = LY.LayerStreamBuffer(E, lay.record_bytes)
    for layer in range(n_layers):
        st = LY.stream_layer(pool, layer, logits[layer], x, sc, lb, L.SCR_W_NVFP4, shape=(k, H, I))
        torch.cuda.synchronize()
        assert torch.equal(bufs[layer]["y"], st["y"]), f"layer {layer}: staged equals stream bit for bit"
        # every output element against the oracle
        lg = W.logits_normal(seed, layer, T, E)
        ids, w = route_topk_softmax(lg, k)
        flush(f"layer {layer}: oracle over all {T} tokens")
        y_ref = moe_layer(bf16_bits_to_f64(xb), ids, w, lambda e: src.f64(layer * E + e))
        y = bufs[layer]["y"].cpu().numpy()
        err = rel_max_err(y, y_ref)
        flush(f"layer {layer}: rel max err over every element {err:.3e}")
        assert err <= 5e-2


@pytest.mark.parametrize("entry", ["kernel", "dma"])
@pytest.mark.parametrize("pattern", ["alternating", "ragged"])
def test_stage_rows_copies_every_run_across_launches(pattern, entry):
    """stage_rows_async (the copy kernel) and stage_rows_dma_async (one
    hipMemcpyAsync per run) move each run of a layer's non-resident experts from
    the pinned pool into the staging buffer at e * record_bytes and nothing
    else: 256 single-record runs (more than one launch's worth of run
    descriptors) or runs of mixed length, checked byte for byte against the
    host records, with the staging buffer's other records left untouched."""
    import slot_cache_routed_amd._lib as L
    import slot_cache_routed_amd.layer as LY
    NL, E, rec = 2, 512, 4096 + 256
    layer = 1
    flush(f"stage_rows runs: {pattern}, {entry}")
    pool = LY.HostPool(NL, E, rec, NL * E)
    g = np.random.default_rng(17)
    pool.records.copy_(torch.from_numpy(g.integers(0, 256, NL * E * rec, dtype=np.uint8)))
    if pattern == "alternating":
        runs = [(layer, e, 1) for e in range(0, E, 2)]
    else:
        runs, e = [], 0
        while e < E:
            n = int(g.integers(1, 9))
            if g.random() < 0.6:
                runs.append((layer, e, min(n, E - e)))
            e += n + int(g.integers(1, 4))
        runs.append((0, 3, 5))          # another layer's run: skipped for this layer
    arr = (L.Run * len(runs))(*[L.Run(*r) for r in runs])
    dst = torch.full((E * rec,), 0xA5, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    stage = L.stage_rows_async if entry == "kernel" else L.stage_rows_dma_async
    stage(pool.desc, arr, len(runs), layer, dst, s, None, None)
    torch.cuda.synchronize()
    got = dst.cpu().view(E, rec)
    staged = np.zeros(E, bool)
    for (l, b, c) in runs:
        if l == layer:
            staged[b:b + c] = True
    for e in range(E):
        if staged[e]:
            assert torch.equal(got[e], pool.key_record(layer * E + e)), e
        else:
            assert bool((got[e] == 0xA5).all()), e
    assert staged.sum() > 0
