"""GPU parity of the activation-quantising formats (FreeToken PR #676,
Solution, fourth bullet: activations quantised under the max of the routed
layer's input scales; Tests, fourth bullet: the layer's 2.0 / 3.0, never the
bank's 9.0).

* the quantisers (scr_quantize_fp8, scr_quantize_nvfp4) bit-exact against
  the oracle's codes;
* W4A8 (MXFP4 weights, FP8 activations) and W4A4 (NVFP4 weights, NVFP4
  activations) layers: x's codes in the workspace bit-exact; every h code the
  oracle's decision or, where the oracle's h lies within the GEMM's rounding
  of a decision point, its neighbour; y against the oracle (whole output)
  within the FP4 tolerance, both as the oracle computes it and with the
  device's side of those near-tie decisions; slot path bit-identical to the
  whole-layer path;
* the layer-view workload (600 tokens, 8 experts over an 1100-slot bank of
  other layers' experts): a_scale is the layer's 3.0, the output is the
  oracle's under 3.0, and a bank-sized scale array (9.0) would change it."""
import numpy as np
import pytest
import torch

import workloads as W
from helpers import ExpertSource, fill_pool, flush, rel_max_err, wdtype_code
from oracle import (dequant_fp8_static, dequant_nvfp4_act, e2m1_encode_array, e2m1_value, e4m3_value,
                    layer_activation_scales,
                    moe_layer_w4a4, moe_layer_w4a8, quantize_fp8_static, quantize_nvfp4_act, route_topk_softmax)
from oracle.mlp import bf16_bits_to_f64

pytestmark = pytest.mark.gpu

TOL_FP4 = 5e-2     # max |y - y_ref| / rms(y_ref)
E4M3 = np.array([0.0 if (c & 0x7F) == 0x7F else e4m3_value(c) for c in range(256)])
E2M1 = np.array([e2m1_value(c) for c in range(16)])


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _inputs(rows, cols, seed):
    g = np.random.default_rng(seed)
    x = g.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp2(g.integers(-6, 6, size=(rows, 1))).astype(np.float32)   # row magnitudes apart
    x[0, :16] = 0.0                                                       # an all-zero block
    if cols >= 64:
        x[-1, 16:32] = [5000.0, -3e-4, 1e-5, -1e-5] * 4                   # saturation, zero codes, signs
        x[-1, 32:48] = 1e-6                                               # a block whose scale rounds to 0
    return W.f32_to_bf16_bits(x)


@pytest.mark.parametrize("rows,cols", [(1, 16), (37, 256), (128, 2048), (4096, 2048)])
def test_quantize_fp8_is_bit_exact(rows, cols):
    import slot_cache_routed_amd._lib as L
    bits = _inputs(rows, cols, rows + cols)
    scales = np.array([0.5, 1.75, 0.25, 1.0], np.float32)               # the max, 1.75, is not first
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    L.quantize_fp8(_dev(bits.view(np.int16)), rows, cols, _dev(scales), 4, q, _stream())
    torch.cuda.synchronize()
    want = quantize_fp8_static(bf16_bits_to_f64(bits).astype(np.float32), 1.75)
    got = q.cpu().numpy()
    assert np.array_equal(got, want), f"{(got != want).sum()} codes differ"


@pytest.mark.parametrize("rows,cols", [(1, 16), (37, 256), (128, 2048), (4096, 2048)])
def test_quantize_nvfp4_is_bit_exact(rows, cols):
    import slot_cache_routed_amd._lib as L
    bits = _inputs(rows, cols, 3 * rows + cols)
    scales = np.array([0.125, 0.3, 0.2], np.float32)
    q = torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda")
    bs = torch.empty((rows, cols // 16), dtype=torch.uint8, device="cuda")
    L.quantize_nvfp4(_dev(bits.view(np.int16)), rows, cols, _dev(scales), 3, q, bs, _stream())
    torch.cuda.synchronize()
    codes, bsc = quantize_nvfp4_act(bf16_bits_to_f64(bits).astype(np.float32), np.float32(0.3))
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    assert np.array_equal(bs.cpu().numpy(), bsc), "block scale codes"
    got = q.cpu().numpy()
    assert np.array_equal(got, packed), f"{(got != packed).sum()} code bytes differ"


# ------------------------------------------------------------------ layers

def _layer(mode, T, E, k, H, I, seed, sc, sc2, S=None, fill=None):
    import slot_cache_routed_amd.layer as LY
    wd = {"w4a8": "mxfp4_a8", "w4a4": "nvfp4_a4"}[mode]
    code = wdtype_code(wd)
    lay = LY.record_layout(code, H, I)
    src = ExpertSource(seed, H, I, wd)
    NL = 2 if fill is not None else 1
    pool = LY.HostPool(NL, E, lay.record_bytes, E, payload_of=lambda key: key % E)
    fill_pool(pool, src, lay, range(E))
    lg = W.logits_normal(seed, 0, T, E)
    xb = W.f32_to_bf16_bits(W.activations_normal(seed, T, H))
    bank = LY.Bank(S or E, NL, E, code, lay.record_bytes)
    if fill is not None:
        bank.load_fill(fill)
    d = LY.demand_layer(bank, pool, 0, _dev(lg), _dev(xb.view(np.int16)), _dev(sc), width=min(E, 64),
                        shape=(k, H, I), fused=True, down_input_scale=_dev(sc2))
    lb = LY.LayerStreamBuffer(E, lay.record_bytes)
    st = LY.stream_layer(pool, 0, _dev(lg), _dev(xb.view(np.int16)), _dev(sc), lb, code, shape=(k, H, I),
                         down_input_scale=_dev(sc2))
    torch.cuda.synchronize()
    return dict(src=src, lg=lg, xb=xb, d=d, st=st, bank=bank, pool=pool, lay=lay, code=code)


def _ws(mode, buf, T, H, I):
    """x's activation values and h's codes/values from the forward's workspace
    (the layout scr_moe_workspace describes: h, per-route rows, their exponent
    bytes (one per 32 columns), flags, scales, then for W4A4 the fp16 x).  h
    has R + min(R, E_layer) * 15 rows (block 16)."""
    al = lambda v: (v + 255) // 256 * 256
    ws = buf["moe_ws"].cpu().numpy()
    R = T * buf.k
    rows = (R + min(R, buf.E) * 15 + 15) // 16 * 16
    if mode == "w4a8":
        h_off = al(T * H)
        o_off = al(h_off + rows * I)
        return ws[:T * H].reshape(T, H), ws[h_off:h_off + rows * I].reshape(rows, I)
    o_off = al(rows * I * 2)
    oe_off = al(o_off + R * H * 2)
    flags_off = al(oe_off + R * (H // 32))
    act_off = al(flags_off + R * 4)
    x16_off = al(act_off + 8)
    h = ws[:rows * I * 2].view(np.float16).reshape(rows, I)
    x16 = ws[x16_off:x16_off + T * H * 2].view(np.float16).reshape(T, H)
    return x16, h


def _check_layer(mode, env, T, E, k, H, I, sc, sc2, end_to_end=True):
    """end_to_end=False: y is asserted against the oracle with the device's
    side of the near-tie h decisions only (each one checked valid above); the
    plain oracle distance is reported.  At millions of h values a few land
    within the GEMM's fp32 rounding of an e2m1 decision point, and one such
    flip moves an output element by up to about a third of its block's
    magnitude through W2."""
    d = env["d"]
    src = env["src"]
    y = d["y"].float().cpu().numpy()
    ids, w = route_topk_softmax(env["lg"], k)
    x = bf16_bits_to_f64(env["xb"])
    a1, a2 = layer_activation_scales(sc, sc2)
    assert d["a_scale"].cpu().numpy().tolist() == [float(a1), float(a2)]
    xws, hws = _ws(mode, d, T, H, I)
    # x: bit-exact
    if mode == "w4a8":
        xq_ref = quantize_fp8_static(x.astype(np.float32), a1)
        assert np.array_equal(xws, xq_ref), f"{(xws != xq_ref).sum()} x codes differ"
        xhat = dequant_fp8_static(xq_ref, a1)
    else:
        xc, xs = quantize_nvfp4_act(x.astype(np.float32), a1)
        xhat = dequant_nvfp4_act(xc, xs, a1)
        assert np.array_equal(xws.astype(np.float64) * float(a1), xhat), "x's decoded NVFP4 values differ"
    # h of every route, the oracle's in fp64 and the size of the GEMM's
    # rounding of it, B = |x||G| |u| + |g| |x||U|
    sr = d["sorted_routes"].cpu().numpy()
    pos = np.nonzero((sr >= 0) & (sr < T * k))[0]
    routes = sr[pos]
    e_of = ids.reshape(-1)[routes]
    h_ref = np.zeros((len(pos), I))
    bnd = np.zeros((len(pos), I))
    for e in np.unique(e_of):
        sel = np.nonzero(e_of == e)[0]
        w13, _ = src.f64(int(e))
        xt = xhat[routes[sel] // k]
        g, u = xt @ w13[:I].T, xt @ w13[I:].T
        h_ref[sel] = g / (1 + np.exp(-g)) * u
        bnd[sel] = (np.abs(xt) @ np.abs(w13[:I]).T) * np.abs(u) + np.abs(g) * (np.abs(xt) @ np.abs(w13[I:]).T)
    delta = 2.0 ** -14 * bnd + 1e-30
    # the device's h values, and the set of values the oracle's rule gives to
    # any h within delta of the oracle's
    if mode == "w4a8":
        h_dev = E4M3[hws[pos]] * float(a2)
        lo = dequant_fp8_static(quantize_fp8_static((h_ref - delta).astype(np.float32), a2), a2)
        hi = dequant_fp8_static(quantize_fp8_static((h_ref + delta).astype(np.float32), a2), a2)
        h_or = dequant_fp8_static(quantize_fp8_static(h_ref.astype(np.float32), a2), a2)
        ok = (h_dev >= np.minimum(lo, hi)) & (h_dev <= np.maximum(lo, hi))
    else:
        h_dev = hws[pos].astype(np.float64) * float(a2)
        h_or = dequant_nvfp4_act(*quantize_nvfp4_act(h_ref.astype(np.float32), a2), a2)
        # per 16-column block: the device's block may also follow an amax
        # within delta of the oracle's; check each element against the
        # roundings of h -+ delta under both candidate block scales
        ok = np.zeros_like(h_dev, dtype=bool)
        for sgn in (-1.0, 0.0, 1.0):
            hv = (h_ref + sgn * delta).astype(np.float32)
            c, s_ = quantize_nvfp4_act(hv, a2)
            ok |= dequant_nvfp4_act(c, s_, a2) == h_dev
            # the same block scale with the element rounded from the other side
            for sg2 in (-1.0, 1.0):
                he = (h_ref + sg2 * delta).astype(np.float32)
                blk = np.repeat(E4M3[s_], 16, axis=1)
                den = blk.astype(np.float32) * np.float32(a2)
                rcp = np.where(den > 0, np.float32(1.0) / np.where(den > 0, den, np.float32(1.0)), np.float32(0.0))
                mag = e2m1_encode_array((he * rcp.astype(np.float32)).astype(np.float32)) & 7
                # the decoded value is the exact product e2m1 * block * a2 (as
                # dequant_nvfp4_act forms it), not e2m1 times the fp32 block * a2
                ok |= (E2M1[mag] * np.sign(he) * blk * float(a2)) == h_dev
    n_diff = int((h_dev != h_or).sum())
    flush(f"{mode} {T}x{E} k={k} H={H} I={I}: h values differing from the oracle's: {n_diff} of {h_or.size}")
    assert ok.all(), f"{(~ok).sum()} h values are no rounding of a value near the oracle's h"
    # y: against the oracle, and against the oracle's down of the device's h
    if mode == "w4a8":
        y_ref = moe_layer_w4a8(x, ids, w, src.f64, sc, sc2)
    else:
        y_ref = moe_layer_w4a4(x, ids, w, src.f64, sc, sc2)
    o = np.zeros((T * k, H))
    for e in np.unique(e_of):
        sel = np.nonzero(e_of == e)[0]
        _, w2 = src.f64(int(e))
        o[routes[sel]] = h_dev[sel] @ w2.T
    y_dn = np.zeros((T, H))
    for j in range(k):
        y_dn += w[:, j:j + 1] * o[j::k]
    err, err_dn = rel_max_err(y, y_ref), rel_max_err(y, y_dn)
    flush(f"{mode} {T}x{E}: rel max err vs the oracle = {err:.3e}, with the device's near-tie h = {err_dn:.3e}")
    assert err_dn <= TOL_FP4
    if end_to_end:
        assert err <= TOL_FP4
    assert torch.equal(d["y"], env["st"]["y"]), "slot path equals the whole-layer path bit for bit"
    return y, y_ref


# few rows per expert (16-row passes) and many (112-row passes, a second pass
# for the fullest buckets), I = 512 resident in down and H streamed
@pytest.mark.parametrize("mode", ["w4a8", "w4a4"])
@pytest.mark.parametrize("T,E,k,H,I", [(64, 32, 4, 512, 512), (384, 16, 4, 512, 512), (500, 12, 3, 1024, 512),
                                       (96, 8, 2, 2048, 512), (200, 16, 4, 512, 1024),
                                       # K blocks in pairs: the two-buffer kernels (I = 768 streams
                                       # h through them; I = 256 keeps it resident)
                                       (384, 16, 4, 512, 768), (384, 16, 4, 512, 256)])
def test_activation_quantising_layer_vs_oracle_and_stream(mode, T, E, k, H, I):
    g = np.random.default_rng(T + E)
    sc = (0.5 + g.random(E)).astype(np.float32)
    sc2 = (0.25 + g.random(E)).astype(np.float32)
    env = _layer(mode, T, E, k, H, I, T + E, sc, sc2)
    _check_layer(mode, env, T, E, k, H, I, sc, sc2)


@pytest.mark.parametrize("mode", ["w4a8", "w4a4"])
def test_layer_view_takes_the_layers_scales_not_the_banks(mode):
    """600 tokens, top-2 over a layer of 8 experts, an 1100-slot bank filled
    with other layers' experts whose scales are 9.0: the forward quantises under
    the layer's 3.0 (even experts 2.0, odd 3.0), matches the oracle under 3.0,
    and differs from what a bank-sized array of 9.0 gives."""
    import slot_cache_routed_amd.layer as LY
    T, E, k, H, I, S = 600, 8, 2, 2048, 512, 1100
    sc = W.c3_input_scales(E)
    fill = W.bank_prefilled(3, S, 2, E, 8, exclude_layer=0)
    env = _layer(mode, T, E, k, H, I, 3, sc, sc, S=S, fill=fill)
    d = env["d"]
    assert d.cfg_used.as_tuple() == LY.L.tile_config(T, k, E, env["code"]).as_tuple()
    y, y_ref = _check_layer(mode, env, T, E, k, H, I, sc, sc)
    assert d["a_scale"].cpu().numpy().tolist() == [3.0, 3.0]
    # the same forward handed a slot-indexed scale array (every slot 9.0)
    bank_scales = _dev(np.full(S, 9.0, np.float32))
    view = LY.make_view(0, S, k, H, I, env["code"], S, env["bank"].row_table, bank_scales, bank_scales)
    buf9 = LY.LayerBuffers(T, S, k, H, I, S, env["code"])
    for key in ("topk_w", "sorted_routes", "active_buckets", "active_block_begin", "n_active"):
        buf9.t[key] = d[key]
    LY.forward(buf9, view, _dev(env["xb"].view(np.int16)))
    torch.cuda.synchronize()
    assert buf9["a_scale"].cpu().numpy().tolist() == [9.0, 9.0]
    y9 = buf9["y"].float().cpu().numpy()
    assert not np.array_equal(y9, y), "the bank's scales change the quantised output"
    ids, w = route_topk_softmax(env["lg"], k)
    x = bf16_bits_to_f64(env["xb"])
    fn = moe_layer_w4a8 if mode == "w4a8" else moe_layer_w4a4
    y9_ref = fn(x, ids, w, env["src"].f64, [9.0], [9.0])
    e9, e3 = rel_max_err(y9, y9_ref), rel_max_err(y9, y_ref)
    flush(f"{mode} layer view: under 9.0 vs the oracle under 9.0 {e9:.3e}, vs the oracle under 3.0 {e3:.3e}")
    assert e9 <= TOL_FP4 and e9 < e3


def test_activation_quantising_forward_rejects_what_it_cannot_run():
    import slot_cache_routed_amd._lib as L
    import slot_cache_routed_amd.layer as LY
    rows = torch.zeros(4, dtype=torch.int64, device="cuda")
    sc = torch.ones(4, dtype=torch.float32, device="cuda")
    x = torch.zeros((8, 256), dtype=torch.int16, device="cuda")
    for code in (L.SCR_W_MXFP4_A8, L.SCR_W_NVFP4_A4):
        view = LY.make_view(0, 4, 2, 256, 512, code, 4, rows, sc)          # H = 256: off the tiling
        buf = LY.LayerBuffers(8, 4, 2, 256, 512, 4, code)
        with pytest.raises(L.ScrError) as ei:
            LY.forward(buf, view, x)
        assert ei.value.code == L.SCR_ENOTSUP
        view = L.RoutedExperts(0, 4, 2, 512, 512, code, 4, rows.data_ptr(), sc.data_ptr(), None)
        buf = LY.LayerBuffers(8, 4, 2, 512, 512, 4, code)
        with pytest.raises(L.ScrError) as ei:                              # no down input scales
            LY.forward(buf, view, torch.zeros((8, 512), dtype=torch.int16, device="cuda"))
        assert ei.value.code == L.SCR_EINVAL
    torch.cuda.synchronize()
