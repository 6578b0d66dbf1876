"""GPU parity of the W4A8 path: MXFP8 quantisation of activations bit-exact
against the oracle's OCP MX rule, and the routed layer with MXFP4 weights and
MXFP8 activations on the block-scaled MFMA against the oracle's W4A8 layer;
slot path bit-identical to the whole-layer path."""
import numpy as np
import pytest
import torch

import workloads as W
from helpers import flush, rel_max_err
from oracle import dequant_mxfp8, e4m3_value, moe_layer_w4a8, quantize_mxfp8, route_topk_softmax
from oracle.lowbit import _e4m3_encode_array
from oracle.mlp import bf16_bits_to_f64

pytestmark = pytest.mark.gpu

TOL_DOWN = 5e-2   # max |y - y_ref| / rms(y_ref), y_ref = the oracle's down of the device's h (bf16 per-route rows, as for every narrow format)


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("rows,cols", [(1, 32), (37, 256), (128, 2048), (4096, 2048)])
def test_quantize_mxfp8_is_bit_exact(rows, cols):
    import slot_cache_routed_amd._lib as L
    g = np.random.default_rng(rows * 7 + cols)
    x = g.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp2(g.integers(-30, 30, size=(rows, 1))).astype(np.float32)    # row magnitudes far apart
    x[0, :32] = 0.0                                                         # an all-zero block
    if cols >= 64:
        x[-1, 32:64] = g.choice([448.0, -447.0, 1e-3, 3.0], size=32)        # saturation and tiny values
    bits = W.f32_to_bf16_bits(x)
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    s = torch.empty((rows, cols // 32), dtype=torch.uint8, device="cuda")
    L.quantize_mxfp8(_dev(bits.view(np.int16)), rows, cols, q, s, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    rq, rs = quantize_mxfp8(bf16_bits_to_f64(bits))
    assert np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(q.cpu().numpy(), rq)


def _layer(T, E, k, H, I, seed, S=None):
    import slot_cache_routed_amd.layer as LY
    import slot_cache_routed_amd._lib as L
    from helpers import ExpertSource, fill_pool
    lay = LY.record_layout(L.SCR_W_MXFP4_A8, H, I)
    src = ExpertSource(seed, H, I, "mxfp4_a8")
    pool = LY.HostPool(1, E, lay.record_bytes, E)
    fill_pool(pool, src, lay, range(E))
    lg = W.logits_normal(seed, 0, T, E)
    xb = W.f32_to_bf16_bits(W.activations_normal(seed, T, H))
    sc = _dev(np.ones(E, np.float32))
    out = {}
    for wcode in (L.SCR_W_MXFP4_A8, L.SCR_W_MXFP4):
        bank = LY.Bank(S or E, 1, E, wcode, lay.record_bytes)
        out[wcode] = LY.demand_layer(bank, pool, 0, _dev(lg), _dev(xb.view(np.int16)), sc, width=min(E, 64),
                                     shape=(k, H, I), fused=True)
    lb = LY.LayerStreamBuffer(E, lay.record_bytes)
    st = LY.stream_layer(pool, 0, _dev(lg), _dev(xb.view(np.int16)), sc, lb, L.SCR_W_MXFP4_A8, shape=(k, H, I))
    torch.cuda.synchronize()
    return src, lg, xb, out, st


def quantize_codes_at(v, scale):
    """e4m3 codes of v under given block scales (the oracle's rounding rule)."""
    return _e4m3_encode_array(v / scale)


def _ws_views(buf, T, H, I):
    """The MXFP8 codes and scales of x and h in the forward's workspace
    (x codes, x scales, h codes, h scales, each 256-byte aligned)."""
    al = lambda v: (v + 255) // 256 * 256
    ws = buf["moe_ws"].cpu().numpy()
    rows = buf.cap
    xs_off = al(T * H)
    h_off = al(xs_off + T * H // 32)
    hs_off = al(h_off + rows * I)
    return (ws[:T * H].reshape(T, H), ws[xs_off:xs_off + T * H // 32].reshape(T, H // 32),
            ws[h_off:h_off + rows * I].reshape(rows, I), ws[hs_off:hs_off + rows * I // 32].reshape(rows, I // 32))


# few rows per expert (16-row passes) and many (112-row passes, a second pass
# for the fullest buckets), K = I resident in down and H streamed
@pytest.mark.parametrize("T,E,k,H,I", [(64, 32, 4, 512, 512), (384, 16, 4, 512, 512), (500, 12, 3, 1024, 512),
                                       (96, 8, 2, 2048, 512)])
def test_w4a8_layer_vs_oracle_and_stream(T, E, k, H, I):
    """h is quantised from the GEMM's fp32 accumulation, the oracle's from
    fp64, so an h value within rounding distance of an e4m3 decision point can
    take the neighbouring code.  Checked: x's codes bit-exact; every h code
    the oracle's, or its neighbour where the oracle's h sits within 2^-12 of
    a code midpoint or its block maximum within 2^-12 of a power of two; and
    y against the oracle's down projection of the device's own h (which
    isolates the down GEMM and the combine) to the narrow formats' tolerance.  The end-
    to-end distance to the W4A8 oracle (which carries the rare flipped h codes
    through W2) and to the W4A16 output are reported."""
    import slot_cache_routed_amd._lib as L
    src, lg, xb, out, st = _layer(T, E, k, H, I, seed=T + E)
    buf = out[L.SCR_W_MXFP4_A8]
    y = buf["y"].float().cpu().numpy()
    ids, w = route_topk_softmax(lg, k)
    x = bf16_bits_to_f64(xb)
    xq, xs, hq, hs = _ws_views(buf, T, H, I)
    rq, rs = quantize_mxfp8(x)
    assert np.array_equal(xq, rq) and np.array_equal(xs, rs)
    xhat = dequant_mxfp8(rq, rs)
    sr = buf["sorted_routes"].cpu().numpy()
    pos = np.nonzero((sr >= 0) & (sr < T * k))[0]
    routes = sr[pos]
    # the oracle's h of every route with the first-order size of the GEMM's
    # rounding in it, B = |x||G| |u| + |g| |x||U|
    h_ref = np.zeros((len(pos), I))
    bnd = np.zeros((len(pos), I))
    for e in np.unique(ids.reshape(-1)[routes]):
        sel = np.nonzero(ids.reshape(-1)[routes] == e)[0]
        w13, _ = src.f64(int(e))
        xt = xhat[routes[sel] // k]
        g, u = xt @ w13[:I].T, xt @ w13[I:].T
        h_ref[sel] = g / (1 + np.exp(-g)) * u
        bnd[sel] = (np.abs(xt) @ np.abs(w13[:I]).T) * np.abs(u) + np.abs(g) * (np.abs(xt) @ np.abs(w13[I:]).T)
    hq_ref, hs_ref = quantize_mxfp8(h_ref)
    hq_dev, hs_dev = hq[pos], hs[pos]
    amax = np.max(np.abs(h_ref.reshape(len(pos), I // 32, 32)), axis=2)
    lg2 = np.log2(np.maximum(amax, 1e-300))
    scale_ok = (hs_dev == hs_ref) | (np.abs(lg2 - np.round(lg2)) < 2.0 ** -12)
    assert scale_ok.all(), f"{(~scale_ok).sum()} h block scales differ away from a power of two"
    # every device code is the oracle's rounding (same block scale) of some
    # value within eps * B of the oracle's h; eps = 2^-12, four times the
    # block-scaled MFMA's measured rounding
    same = np.repeat(hs_dev == hs_ref, 32, axis=1)
    sc = np.exp2(hs_dev.astype(np.float64) - 127).repeat(32, axis=1)
    e4 = np.array([e4m3_value(c) for c in range(256)])
    delta = 2.0 ** -12 * bnd
    lo = e4[quantize_codes_at(h_ref - delta, sc)]
    hi = e4[quantize_codes_at(h_ref + delta, sc)]
    v_dev = e4[hq_dev]
    ok = ~same | ((v_dev >= np.minimum(lo, hi)) & (v_dev <= np.maximum(lo, hi)))
    n_diff = int(((e4[hq_dev] != e4[hq_ref]) & same).sum())
    flush(f"w4a8 {T}x{E}: h codes differing from the oracle's: {n_diff} of {hq_ref.size}")
    assert ok.all(), f"{(~ok).sum()} h codes are no rounding of a value near the oracle's h"
    # down + combine from the device's h
    hhat = dequant_mxfp8(hq_dev, hs_dev)
    o = np.zeros((T * k, H))
    for e in np.unique(ids.reshape(-1)[routes]):
        sel = np.nonzero(ids.reshape(-1)[routes] == e)[0]
        _, w2 = src.f64(int(e))
        o[routes[sel]] = hhat[sel] @ w2.T
    y_dn = np.zeros((T, H))
    for j in range(k):
        y_dn += w[:, j:j + 1] * o[j::k]
    err_dn = rel_max_err(y, y_dn)
    y_ref = moe_layer_w4a8(x, ids, w, src.f64)
    err = rel_max_err(y, y_ref)
    y16 = out[L.SCR_W_MXFP4]["y"].float().cpu().numpy()
    flush(f"w4a8 {T}x{E} k={k} H={H} I={I}: rel max err vs the oracle's down of the device h = {err_dn:.3e}, "
          f"vs the W4A8 oracle = {err:.3e}; W4A8 vs W4A16 output: {rel_max_err(y, y16):.3e}")
    assert err_dn <= TOL_DOWN
    assert torch.equal(buf["y"], st["y"]), "slot path equals the whole-layer path bit for bit"


def test_w4a8_rejects_shapes_off_its_tiling():
    import slot_cache_routed_amd._lib as L
    import slot_cache_routed_amd.layer as LY
    rows = torch.zeros(4, dtype=torch.int64, device="cuda")
    sc = torch.ones(4, dtype=torch.float32, device="cuda")
    view = LY.make_view(0, 4, 2, 256, 512, L.SCR_W_MXFP4_A8, 4, rows, sc)
    buf = LY.LayerBuffers(8, 4, 2, 256, 512, 4, L.SCR_W_MXFP4_A8)
    x = torch.zeros((8, 256), dtype=torch.int16, device="cuda")
    with pytest.raises(L.ScrError) as ei:
        LY.forward(buf, view, x)
    assert ei.value.code == L.SCR_ENOTSUP
