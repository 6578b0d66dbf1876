"""GPU parity of the whole routed layer: demand (slot) path against the
oracle, slot path bit-identical to the whole-layer stream path, the layer
view's tiles and scales, NVFP4 decode in the GEMM, and 64-bit row offsets."""
import functools

import numpy as np
import pytest
import torch

import workloads as W
from helpers import ExpertSource, fill_pool, flush, rel_max_err, wdtype_code
from oracle import moe_layer, moe_layer_tokens, route_topk_softmax
from oracle.mlp import bf16_bits_to_f64

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2   # max |y - y_ref| / rms(y_ref)
TOL_FP4 = 5e-2


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@functools.lru_cache(maxsize=None)
def _setup(name, S=None, W_=None, prefill=None, wdtype=None, T=None, E=None, k=None, H=None, I=None, NL=None):
    """Pool, bank and inputs of one workload (cached per process)."""
    import slot_cache_routed_amd.layer as LY
    import slot_cache_routed_amd._lib as L
    cfg = W.CONFIGS.get(name)
    T = T or cfg.T
    E = E or cfg.shape.E
    k = k or cfg.shape.k
    H = H or cfg.shape.H
    I = I or cfg.shape.I
    wd = wdtype or cfg.shape.wdtype
    S = S or cfg.S
    NL = NL or cfg.L
    seed = cfg.seed if cfg else 77
    wcode = wdtype_code(wd)
    lay = LY.record_layout(wcode, H, I)
    src = ExpertSource(seed, H, I, wd)
    flush(f"setup {name}: T={T} E={E} k={k} H={H} I={I} {wd} S={S} layers={NL}")
    pool = LY.HostPool(NL, E, lay.record_bytes, E, payload_of=lambda key: key % E)
    fill_pool(pool, src, lay, range(E))
    if name == "short_prefill_96":
        lg, D = W.logits_with_chosen(seed, T, E, k, 160)
    else:
        lg = W.logits_normal(seed, 0, T, E)
    xb = W.f32_to_bf16_bits(W.activations_normal(seed, T, H))
    return dict(LY=LY, L=L, T=T, E=E, k=k, H=H, I=I, wd=wd, wcode=wcode, S=S, NL=NL, seed=seed, lay=lay, src=src,
                pool=pool, logits=lg, xbits=xb, W=W_ or (cfg.W if cfg else 8), prefill=prefill)


def _bank_for(s, fill=None):
    bank = s["LY"].Bank(s["S"], s["NL"], s["E"], s["wcode"], s["lay"].record_bytes)
    if fill is not None:
        bank.load_fill(fill)
    return bank


def _run_demand(s, bank, input_scale, y_dtype=0, width=None):
    LY = s["LY"]
    return LY.demand_layer(bank, s["pool"], 0, _dev(s["logits"]), _dev(s["xbits"].view(np.int16)),
                           _dev(input_scale), width=width or s["W"], record_stats=False, y_dtype=y_dtype,
                           shape=(s["k"], s["H"], s["I"]))


def _run_stream(s, input_scale, y_dtype=0):
    LY = s["LY"]
    lb = LY.LayerStreamBuffer(s["E"], s["lay"].record_bytes)
    return LY.stream_layer(s["pool"], 0, _dev(s["logits"]), _dev(s["xbits"].view(np.int16)), _dev(input_scale),
                           lb, s["wcode"], y_dtype=y_dtype, shape=(s["k"], s["H"], s["I"]))


def _oracle(s, tokens=None):
    ids, w = route_topk_softmax(s["logits"], s["k"])
    x = bf16_bits_to_f64(s["xbits"])
    if tokens is None:
        return moe_layer(x, ids, w, s["src"].f64), ids, w
    return moe_layer_tokens(x, ids, w, s["src"].f64, tokens), ids, w


def _y(buf):
    torch.cuda.synchronize()
    return buf["y"].float().cpu().numpy()


def test_tiny_layer_demand_vs_oracle_and_stream():
    s = _setup("tiny")
    bank = _bank_for(s)
    sc = np.ones(s["E"], np.float32)
    d = _run_demand(s, bank, sc)
    y = _y(d)
    y_ref, ids, w = _oracle(s)
    assert np.array_equal(d["topk_ids"].cpu().numpy().reshape(ids.shape), ids)
    err = rel_max_err(y, y_ref)
    flush(f"tiny: rel max err vs oracle on the bf16 weights = {err:.3e}")
    assert err <= TOL_BF16
    # against the fp32 originals the difference also includes the bf16 upload
    x = bf16_bits_to_f64(s["xbits"])
    y_f32w = moe_layer(x, ids, w, lambda e: tuple(a.astype(np.float64) for a in s["src"].f32_original(e)))
    flush(f"tiny: rel max err vs fp32 original weights = {rel_max_err(y, y_f32w):.3e}")
    st = _run_stream(s, sc)
    assert torch.equal(d["y"], st["y"]), "slot path equals the whole-layer path bit for bit"


def test_short_prefill_96_demand_path():
    s = _setup("short_prefill_96")
    fill = W.bank_prefilled(s["seed"], s["S"], s["NL"], s["E"], 600, exclude_layer=0)
    bank = _bank_for(s, fill)
    sc = np.ones(s["E"], np.float32)
    d = _run_demand(s, bank, sc)
    y = _y(d)
    nm = d["n_miss"].cpu().numpy().tolist()
    assert nm == [128, 32, 0, 0], nm
    assert np.all(bank.snapshot()["stats"] == 0) and np.all(bank.snapshot()["decode_freq"] == 0)
    flush("short prefill: oracle over 96 tokens")
    y_ref, ids, _ = _oracle(s)
    err = rel_max_err(y, y_ref)
    flush(f"short prefill: rel max err = {err:.3e}")
    assert err <= TOL_BF16
    # the 160 admitted rows hold the pool's bytes
    snap = bank.snapshot()
    for e in np.unique(ids)[:8]:
        slot = snap["key_to_slot"][e]
        assert torch.equal(bank.slot_record(slot).cpu(), s["pool"].key_record(int(e)))
    st = _run_stream(s, sc)
    assert torch.equal(d["y"], st["y"]), "slot path equals the whole-layer path bit for bit"
    # bf16 output mode is the same numbers rounded
    d2 = _run_demand(s, bank, sc, y_dtype=1)
    assert torch.equal(d2["y"].float(), d["y"].to(torch.bfloat16).float())


def test_real_size_chunk_of_200_tokens_admits_its_distinct_experts_in_queries_of_128():
    # FreeToken PR #68's real-size case (200 tokens, top-10, 512 experts, 1,100
    # slots): 2,000 routes, but the LRU only ever sees the chunk's distinct
    # experts, at most 128 per query (handing it the routes was what broke)
    from oracle import SlotBankState, dedup_sorted, ensure_slots
    s = _setup("real_size_200", S=1100, W_=128, wdtype="bf16", T=200, E=512, k=10, H=2048, I=512, NL=3)
    fill = W.bank_prefilled(s["seed"], s["S"], s["NL"], s["E"], 600, exclude_layer=0)
    bank = _bank_for(s, fill)
    sc = np.ones(s["E"], np.float32)
    d = _run_demand(s, bank, sc)
    y = _y(d)
    ids, w = route_topk_softmax(s["logits"], s["k"])
    distinct, nd, _ = dedup_sorted(ids.reshape(-1), s["E"])
    st = SlotBankState.from_fill(fill)
    expect = []
    for q0 in range(0, len(distinct), 128):
        ms, _ = ensure_slots(st, 0, distinct[q0:q0 + 128], False)
        expect.append(len(ms))
    nm = d["n_miss"].cpu().numpy().tolist()
    flush(f"200-token chunk: {nd} distinct experts, misses per query {nm}")
    assert nm == expect and max(nm) <= 128 and len(nm) == 4
    snap = bank.snapshot()
    for key in ("slot_key", "key_to_slot", "slot_stamp"):
        assert np.array_equal(np.asarray(snap[key]), np.asarray(getattr(st, key))), key
    y_ref, _, _ = _oracle(s)
    err = rel_max_err(y, y_ref)
    flush(f"200-token chunk: rel max err over all 200 tokens = {err:.3e}")
    assert err <= TOL_BF16
    st_y = _run_stream(s, sc)
    assert torch.equal(d["y"], st_y["y"]), "slot path equals the whole-layer path bit for bit"


def test_layer_view_sizes_tiles_and_scales_by_the_layer():
    s = _setup("layer_view_600")
    L = s["L"]
    fill = W.bank_prefilled(s["seed"], s["S"], s["NL"], s["E"], s["S"], exclude_layer=0)   # full bank
    bank = _bank_for(s, fill)
    layer_scales = W.c3_input_scales(s["E"])
    d = _run_demand(s, bank, layer_scales)
    y = _y(d)
    want = L.tile_config(600, 2, 8, L.SCR_W_BF16).as_tuple()
    assert d.cfg_used.as_tuple() == want
    assert want != L.tile_config(600, 2, s["S"], L.SCR_W_BF16).as_tuple(), "a bank-sized config would differ"
    assert float(d["a_scale"][0].item()) == 3.0     # the layer's max, not the bank's 9.0
    assert d["n_miss"].cpu().numpy()[0] == 8
    st = _run_stream(s, layer_scales)
    assert torch.equal(d["y"], st["y"])
    y_ref, _, _ = _oracle(s)
    err = rel_max_err(y, y_ref)
    flush(f"layer view 600 tokens: rel max err over all tokens = {err:.3e}")
    assert err <= TOL_BF16


def test_layer_view_one_layer_cache_three_per_query():
    s = _setup("layer_view_600_s8")
    fill = W.bank_prefilled(s["seed"], 8, s["NL"], s["E"], 8, exclude_layer=0)
    bank = _bank_for(s, fill)
    sc = W.c3_input_scales(s["E"])
    d = _run_demand(s, bank, sc, width=3)
    assert d["n_miss"].cpu().numpy().tolist() == [3, 3, 2]
    st = _run_stream(s, sc)
    assert torch.equal(d["y"], st["y"])


# the last two take the wide-tile kernels (I = 512, many rows per expert; at
# 1500 routes over 12 experts some buckets need a second M pass)
# Narrow formats (NVFP4; FP8 with a per-tensor scale; MXFP4 with e8m0 block
# scales): every shape above for each, decoded in the GEMM against the
# oracle's table decode
@pytest.mark.parametrize("wd", ["nvfp4", "fp8", "mxfp4"])
@pytest.mark.parametrize("T,E,k,H,I", [(64, 16, 4, 256, 128), (200, 32, 6, 512, 256), (37, 8, 3, 256, 128),
                                       (384, 16, 4, 512, 512), (500, 12, 3, 1024, 512),
                                       # wide kernels with K blocks in pairs (two activation buffers):
                                       # h streamed (I = 768) and resident (I = 256) in the down
                                       (384, 16, 4, 512, 768), (384, 16, 4, 512, 256),
                                       # hidden sizes that are not multiples of 512 (x's fp16 copy
                                       # for the NVFP4 gate/up takes its strided form)
                                       (64, 16, 4, 768, 128), (300, 12, 3, 640, 256)])
def test_narrow_format_layer_vs_oracle_and_stream(wd, T, E, k, H, I):
    s = _setup(f"{wd}_{T}_{E}", S=2 * E, W_=8, wdtype=wd, T=T, E=E, k=k, H=H, I=I, NL=2)
    bank = _bank_for(s)
    sc = np.ones(E, np.float32)
    d = _run_demand(s, bank, sc)
    y = _y(d)
    y_ref, _, _ = _oracle(s)
    err = rel_max_err(y, y_ref)
    flush(f"{wd} {T}x{E} k={k} H={H} I={I}: rel max err = {err:.3e}")
    assert err <= TOL_FP4
    st = _run_stream(s, sc)
    assert torch.equal(d["y"], st["y"])


def test_bf16_ragged_shapes_vs_oracle():
    # many tiles with a ragged tail of rows per bucket
    s = _setup("ragged", S=100, W_=16, wdtype="bf16", T=333, E=24, k=5, H=384, I=256, NL=3)
    bank = _bank_for(s)
    sc = np.ones(s["E"], np.float32)
    d = _run_demand(s, bank, sc)
    y_ref, _, _ = _oracle(s)
    assert rel_max_err(_y(d), y_ref) <= TOL_BF16
    st = _run_stream(s, sc)
    assert torch.equal(d["y"], st["y"])


def test_bf16_wide_tiles_vs_oracle():
    # about 96 rows per expert with I = 512: the wide-tile kernels in bf16
    s = _setup("wide_bf16", S=40, W_=16, wdtype="bf16", T=384, E=16, k=4, H=512, I=512, NL=2)
    bank = _bank_for(s)
    sc = np.ones(s["E"], np.float32)
    d = _run_demand(s, bank, sc)
    assert d.cfg_used.m_chunk == 112
    y_ref, _, _ = _oracle(s)
    err = rel_max_err(_y(d), y_ref)
    flush(f"bf16 wide 384x16: rel max err = {err:.3e}")
    assert err <= TOL_BF16
    st = _run_stream(s, sc)
    assert torch.equal(d["y"], st["y"])


def test_bf16_wide_tiles_with_k_blocks_in_pairs_vs_oracle():
    # hidden and intermediate 768 (six K blocks each): the wide-tile kernels
    # with two activation buffers in both GEMMs
    s = _setup("wide_bf16_768", S=40, W_=16, wdtype="bf16", T=384, E=16, k=4, H=768, I=768, NL=2)
    bank = _bank_for(s)
    sc = np.ones(s["E"], np.float32)
    d = _run_demand(s, bank, sc)
    assert d.cfg_used.m_chunk == 112
    y_ref, _, _ = _oracle(s)
    err = rel_max_err(_y(d), y_ref)
    flush(f"bf16 wide 384x16 H=I=768: rel max err = {err:.3e}")
    assert err <= TOL_BF16
    st = _run_stream(s, sc)
    assert torch.equal(d["y"], st["y"])


@pytest.mark.parametrize("wd", ["bf16", "nvfp4", "fp8"])
def test_few_experts_with_skewed_routing_vs_oracle(wd):
    """8 experts, top-2, Zipf(1.1)-skewed routing over 2048 tokens: bucket
    sizes from about 200 to 1600 rows, so the pass slices of the wide kernels
    leave some workgroups without a pass and give others several, and the
    down's N chunks go to workgroups of their own; every output against the
    oracle and bit-identical to the stream path."""
    s = dict(_setup(f"skewed_few_{wd}", S=16, W_=8, wdtype=wd, T=2048, E=8, k=2, H=512, I=512, NL=2))
    s["logits"] = W.zipf_gumbel_logits(s["seed"], 0, 0, s["T"], s["E"])
    ids, _ = route_topk_softmax(s["logits"], s["k"])
    counts = np.bincount(ids.reshape(-1), minlength=s["E"])
    assert counts.max() >= 4 * counts.min(), counts
    bank = _bank_for(s)
    sc = np.ones(s["E"], np.float32)
    d = _run_demand(s, bank, sc)
    assert d.cfg_used.m_chunk == 112
    y_ref, _, _ = _oracle(s)
    err = rel_max_err(_y(d), y_ref)
    flush(f"skewed 8 experts {wd}: bucket rows {counts.min()}..{counts.max()}, rel max err = {err:.3e}")
    assert err <= (TOL_BF16 if wd == "bf16" else TOL_FP4)
    st = _run_stream(s, sc)
    assert torch.equal(d["y"], st["y"])


def test_rows_past_32_gib_of_bank():
    """The same expert at slot 0 and at a slot whose byte offset is past 2^35
    gives identical outputs; a zero record gives a different one."""
    import slot_cache_routed_amd.layer as LY
    import slot_cache_routed_amd._lib as L
    H, I, T = 2048, 512, 8
    lay = LY.record_layout(L.SCR_W_BF16, H, I)
    S = (1 << 35) // lay.record_bytes + 2
    far = S - 1
    assert far * lay.record_bytes > (1 << 35)
    src = ExpertSource(91, H, I, "bf16")
    pool = LY.HostPool(1, 1, lay.record_bytes, 1)
    fill_pool(pool, src, lay, [0])
    lg = np.zeros((T, 1), np.float32)
    x = _dev(W.f32_to_bf16_bits(W.activations_normal(91, T, H)).view(np.int16))
    sc = _dev(np.ones(1, np.float32))
    bank = LY.Bank(S, 1, 1, L.SCR_W_BF16, lay.record_bytes)
    outs = []
    for slot, zero in ((0, False), (far, False), (far, True)):
        fill = W.bank_empty(S, 1, 1)
        fill.slot_key[slot] = 0
        fill.slot_stamp[slot] = 1
        fill.clock = 1
        bank.load_fill(fill)
        rec = bank.slot_record(slot)
        if zero:
            rec.zero_()
        else:
            rec.copy_(pool.key_record(0).cuda())
        d = LY.demand_layer(bank, pool, 0, _dev(lg), x, sc, width=1, shape=(1, H, I))
        assert d["n_miss"].cpu().numpy()[0] == 0
        outs.append(_y(d))
        if slot != 0:
            rec.zero_()
    assert np.array_equal(outs[0], outs[1])
    assert not np.array_equal(outs[0], outs[2])
    del bank
    torch.cuda.empty_cache()


@pytest.mark.parametrize("H,I", [(256, 128), (512, 512)])
def test_nvfp4_every_scale_code_and_every_e2m1_code(H, I):
    """Block scales cycling over every finite E4M3 code (subnormals, 448, both
    signs) and uniformly random e2m1 codes (both zeros included): the GEMM's
    in-register decode against the oracle's table decode.  40 tokens over 4
    experts give 20 rows per expert (the 112-row passes); 256 x 128 takes the
    narrow-tile kernel, 512 x 512 the wide one (hardware scale conversion)."""
    import slot_cache_routed_amd.layer as LY
    import slot_cache_routed_amd._lib as L
    from oracle import dequant_nvfp4
    T, E, k = 40, 4, 2
    g = np.random.default_rng(448 + H)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)

    def raw(e):
        def sc(rows, cols):
            n = rows * (cols // 16)
            return np.resize(np.roll(finite, 37 * e), n).reshape(rows, cols // 16).astype(np.uint8)
        return {"w13_q": g.integers(0, 256, size=(2 * I, H // 2), dtype=np.uint8), "w13_s": sc(2 * I, H),
                "w2_q": g.integers(0, 256, size=(H, I // 2), dtype=np.uint8), "w2_s": sc(H, I),
                "g13": np.float32(2.0 ** -7), "g2": np.float32(2.0 ** -9)}
    raws = [raw(e) for e in range(E)]
    lay = LY.record_layout(L.SCR_W_NVFP4, H, I)
    pool = LY.HostPool(1, E, lay.record_bytes, E)
    for e in range(E):
        pool.write_payload(e, LY.pack_record_nvfp4(lay, raws[e]))
    lg = W.logits_normal(31, 0, T, E)
    xb = W.f32_to_bf16_bits(W.activations_normal(31, T, H))
    bank = LY.Bank(E, 1, E, L.SCR_W_NVFP4, lay.record_bytes)
    d = LY.demand_layer(bank, pool, 0, _dev(lg), _dev(xb.view(np.int16)), _dev(np.ones(E, np.float32)), width=4,
                        shape=(k, H, I), fused=True)
    y = _y(d)
    ids, w = route_topk_softmax(lg, k)
    f64 = {e: (dequant_nvfp4(raws[e]["w13_q"], raws[e]["w13_s"], raws[e]["g13"]),
               dequant_nvfp4(raws[e]["w2_q"], raws[e]["w2_s"], raws[e]["g2"])) for e in range(E)}
    y_ref = moe_layer(bf16_bits_to_f64(xb), ids, w, lambda e: f64[e])
    err = rel_max_err(y, y_ref)
    flush(f"nvfp4 every scale code, H={H} I={I}: rel max err = {err:.3e}")
    assert err <= TOL_FP4


@pytest.mark.parametrize("H", [512, 1536])
def test_nvfp4_wide_gate_up_rows_of_every_magnitude(H):
    """The wide NVFP4 gate/up takes x as fp16 scaled per token by a power of
    two.  Tokens whose rows are zero, scaled by 2^-40 or 2^40, or hold one
    element 2^20 or 2^35 above the rest (the rest then fp16 subnormals) each
    match the oracle to the FP4 tolerance relative to their own row, and the
    stream path stays bit-identical.  H = 512 keeps the row in registers
    during its conversion, H = 1536 takes the conversion's general loop."""
    import slot_cache_routed_amd.layer as LY
    import slot_cache_routed_amd._lib as L
    T, E, k, I = 48, 4, 2, 512                  # 24 rows per expert: the wide kernels
    src = ExpertSource(61, H, I, "nvfp4")
    lay = LY.record_layout(L.SCR_W_NVFP4, H, I)
    pool = LY.HostPool(1, E, lay.record_bytes, E)
    fill_pool(pool, src, lay, range(E))
    lg = W.logits_normal(61, 0, T, E)
    x = W.activations_normal(61, T, H).astype(np.float64)
    x[0] = 0.0
    x[1] *= 2.0 ** -40
    x[2] *= 2.0 ** 40
    x[3, 7] = 2.0 ** 20
    x[4, H - 212] = -(2.0 ** 35)
    x[5] *= 2.0 ** -20
    x[5, 0] = 2.0 ** 10
    xb = W.f32_to_bf16_bits(x.astype(np.float32))
    bank = LY.Bank(E, 1, E, L.SCR_W_NVFP4, lay.record_bytes)
    sc = np.ones(E, np.float32)
    d = LY.demand_layer(bank, pool, 0, _dev(lg), _dev(xb.view(np.int16)), _dev(sc), width=4, shape=(k, H, I))
    assert d.cfg_used.m_chunk == 112
    y = _y(d)
    ids, w = route_topk_softmax(lg, k)
    y_ref = moe_layer(bf16_bits_to_f64(xb), ids, w, src.f64)
    assert np.all(y[0] == 0.0)
    for t in range(1, T):
        r = float(np.sqrt(np.mean(y_ref[t] ** 2)))
        err = float(np.max(np.abs(y[t].astype(np.float64) - y_ref[t]))) / r
        if t < 8:
            flush(f"nvfp4 wide row {t}: rms {r:.3e}, rel max err {err:.3e}")
        assert np.isfinite(err) and err <= TOL_FP4, (t, err)
    lb = LY.LayerStreamBuffer(E, lay.record_bytes)
    st = LY.stream_layer(pool, 0, _dev(lg), _dev(xb.view(np.int16)), _dev(sc), lb, L.SCR_W_NVFP4, shape=(k, H, I))
    assert torch.equal(d["y"], st["y"])


@pytest.mark.parametrize("wd", ["bf16", "nvfp4", "fp8", "mxfp4", "mxfp4_a8", "nvfp4_a4"])
def test_full_size_4096_token_layer_in_every_weight_format(wd):
    """The benchmark's 4096-token layer (512 experts, top-10, hidden 2048,
    intermediate 512) in each weight format through the demand path
    (every expert admitted into a 512-slot bank, 40,960 routes aligned by the
    multi-workgroup align, the wide GEMM kernels): bit-identical to the
    whole-layer stream path, and every output element within the oracle's
    tolerance (bf16 2e-2, the 4-bit and 8-bit formats 5e-2; W4A8 and W4A4
    against the oracle's activation-quantising layer under the layer's
    scales, 2.0 / 3.0).  Records alias 64 generated payloads."""
    import slot_cache_routed_amd.layer as LY
    T, E, k, H, I, P, seed = 4096, 512, 10, 2048, 512, 64, 5
    code = wdtype_code(wd)
    src = ExpertSource(seed, H, I, wd)
    lay = LY.record_layout(code, H, I)
    flush(f"full-size layer {wd}: packing {P} records")
    pool = LY.HostPool(1, E, lay.record_bytes, P, payload_of=lambda key: key % P)
    fill_pool(pool, src, lay, range(P))
    lg = W.logits_normal(seed, 0, T, E)
    xb = W.f32_to_bf16_bits(W.activations_normal(seed, T, H))
    sc_h = W.c3_input_scales(E)
    sc = _dev(sc_h)
    bank = LY.Bank(E, 1, E, code, lay.record_bytes)
    d = LY.demand_layer(bank, pool, 0, _dev(lg), _dev(xb.view(np.int16)), sc, width=128, shape=(k, H, I))
    torch.cuda.synchronize()
    assert d["n_miss"].cpu().numpy().tolist() == [128, 128, 128, 128]
    assert d.cfg_used.m_chunk == 112
    lb = LY.LayerStreamBuffer(E, lay.record_bytes)
    st = LY.stream_layer(pool, 0, _dev(lg), _dev(xb.view(np.int16)), sc, lb, code, shape=(k, H, I))
    torch.cuda.synchronize()
    assert torch.equal(d["y"], st["y"]), "slot path equals the whole-layer path bit for bit"
    ids, w = route_topk_softmax(lg, k)
    x = bf16_bits_to_f64(xb)
    wf = lambda e: src.f64(e % P)
    flush(f"full-size layer {wd}: oracle over all {T} tokens")
    if wd in ("mxfp4_a8", "nvfp4_a4"):
        # x's codes bit-exact, every h value valid, y against the oracle with
        # the device's side of the near-tie h decisions (the plain distance,
        # which a handful of those flips among 21M h values dominates, is
        # reported)
        import test_gpu_actquant as A

        class _Src:
            f64 = staticmethod(wf)
        A._check_layer("w4a8" if wd == "mxfp4_a8" else "w4a4", dict(src=_Src, lg=lg, xb=xb, d=d, st=st),
                       T, E, k, H, I, sc_h, sc_h, end_to_end=False)
        return
    y_ref = moe_layer(x, ids, w, wf)
    err = rel_max_err(_y(d), y_ref)
    flush(f"full-size layer {wd}: rel max err over every element = {err:.3e}")
    assert err <= (TOL_BF16 if wd == "bf16" else TOL_FP4)
    del bank, lb, pool
    torch.cuda.empty_cache()


@pytest.mark.parametrize("wd", ["bf16", "nvfp4"])
def test_forward_at_the_largest_token_count(wd):
    """T * H just below 2^31, the forward's bound (T = 524,287 tokens of hidden
    4096, so x alone is 4 GiB and the activation byte offsets pass 2^31), over
    a layer of 8 experts with top-1: about 65,500 rows per expert, so the wide
    kernels deal each bucket's 112-row passes to many workgroups.  NVFP4 also
    reads its 4 GiB fp16 copy of x, whose byte offsets approach 2^32.  The
    first, middle and last tokens and a seeded sample are compared with the
    oracle."""
    import slot_cache_routed_amd.layer as LY
    import slot_cache_routed_amd._lib as L
    E, k, H, I, seed = 8, 1, 4096, 512, 13
    T = (1 << 31) // H - 1
    code = wdtype_code(wd)
    src = ExpertSource(seed, H, I, wd)
    lay = LY.record_layout(code, H, I)
    flush(f"largest token count: {wd} T={T} H={H} I={I} E={E} k={k}")
    lb = LY.LayerStreamBuffer(E, lay.record_bytes)
    for e in range(E):
        rec = LY.pack_record_nvfp4(lay, src.raw(e)) if wd == "nvfp4" else LY.pack_record_bf16(lay, *src.raw(e))
        lb.data[e * lay.record_bytes:(e + 1) * lay.record_bytes].copy_(torch.from_numpy(rec))
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, size=T).astype(np.int32)
    b = LY.LayerBuffers(T, E, k, H, I, E, code)
    b["topk_ids"].copy_(torch.from_numpy(ids))
    b["topk_w"].fill_(1.0)
    # x drawn on the device (4 GiB), in row blocks, from a seeded generator
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    for r0 in range(0, T, 1 << 16):
        r1 = min(T, r0 + (1 << 16))
        x[r0:r1] = torch.randn((r1 - r0, H), generator=g, device="cuda").to(torch.bfloat16)
    LY.align(b, None, 0)
    sc = torch.ones(E, dtype=torch.float32, device="cuda")
    view = LY.make_view(0, E, k, H, I, code, E, lb.row_table, sc)
    cfg = LY.forward(b, view, x)
    torch.cuda.synchronize()
    assert cfg.m_chunk == 112
    tokens = np.unique(np.concatenate([[0, 1, T // 2, T - 3, T - 2, T - 1], rng.integers(0, T, size=26)]))
    sel = torch.from_numpy(tokens).cuda()
    xs = bf16_bits_to_f64(x[sel].view(torch.int16).cpu().numpy().view(np.uint16))
    y = b["y"][sel].cpu().numpy()
    y_ref = moe_layer_tokens(xs, ids[tokens].reshape(-1, 1), np.ones((tokens.size, 1)), src.f64, range(tokens.size))
    err = rel_max_err(y, y_ref)
    flush(f"largest token count: {wd} rel max err over {tokens.size} tokens = {err:.3e}")
    assert err <= (TOL_BF16 if wd == "bf16" else TOL_FP4)
    del x, b, lb
    torch.cuda.empty_cache()


@pytest.mark.parametrize("k", [24, 32])
def test_top_k_past_sixteen(k):
    """k above 16: the combine sums a token's ranks in groups of 16 (the second
    group partly clamped), still in rank order; against the oracle and the
    stream path."""
    s = _setup(f"topk_{k}", S=96, W_=32, wdtype="bf16", T=40, E=48, k=k, H=256, I=128, NL=2)
    bank = _bank_for(s)
    sc = np.ones(s["E"], np.float32)
    d = _run_demand(s, bank, sc)
    y_ref, _, _ = _oracle(s)
    err = rel_max_err(_y(d), y_ref)
    flush(f"top-{k}: rel max err = {err:.3e}")
    assert err <= TOL_BF16
    st = _run_stream(s, sc)
    assert torch.equal(d["y"], st["y"])


def test_forward_with_no_tokens_launches_nothing():
    import slot_cache_routed_amd.layer as LY
    import slot_cache_routed_amd._lib as L
    rows = torch.zeros(4, dtype=torch.int64, device="cuda")
    sc = torch.ones(4, dtype=torch.float32, device="cuda")
    view = LY.make_view(0, 4, 2, 256, 128, L.SCR_W_BF16, 4, rows, sc)
    y = torch.full((1, 256), 7.0, device="cuda")
    cfg = L.grouped_moe_forward(view, 0, 0, 0, 0, 0, 0, 0, y, L.SCR_Y_F32, 0, 0, None,
                                torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
