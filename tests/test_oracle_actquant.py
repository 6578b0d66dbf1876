"""Pins for the activation quantisers and the quantising layers of the oracle
(CPU): hand-worked codes and layers, a brute-force rounding check, exact round
trips, scaling invariance, locality, and the dependence on the layer's input
scales only through their maxima."""
import numpy as np
import pytest

from conftest import read_golden
from oracle import (dequant_fp8_static, dequant_nvfp4_act, e2m1_encode_array, e2m1_value, e4m3_value,
                    layer_activation_scales, moe_layer, moe_layer_w4a4, moe_layer_w4a8, quantize_fp8_static,
                    quantize_nvfp4_act)

E2M1 = np.array([e2m1_value(c) for c in range(8)])


def test_fp8_static_codes_worked_by_hand():
    rows = [r for r in read_golden("act_quant_worked_example.txt") if r[0] == "fp8"]
    assert len(rows) == 8
    for _, s, v, code, dec in rows:
        c = quantize_fp8_static(np.array([float(v)]), float(s))
        assert int(c[0]) == int(code, 16), (v, c)
        assert dequant_fp8_static(c, float(s))[0] == float(dec)


def test_nvfp4_activation_codes_worked_by_hand():
    g = read_golden("act_quant_worked_example.txt")
    el = [r for r in g if r[0] == "nv"]
    bl = [r for r in g if r[0] == "nvblock"]
    v = np.zeros((3, 32), np.float32)
    for _, _, r, c, val, _, _ in el:
        v[int(r), int(c)] = float(val)
    codes, scales = quantize_nvfp4_act(v, 0.5)
    dec = dequant_nvfp4_act(codes, scales, 0.5)
    listed = np.zeros_like(v, dtype=bool)
    for _, _, r, c, _, code, d in el:
        r, c = int(r), int(c)
        listed[r, c] = True
        assert int(codes[r, c]) == int(code, 16), (r, c, codes[r, c])
        assert dec[r, c] == float(d), (r, c, dec[r, c])
    assert np.all(dec[~listed] == 0.0)
    for _, _, r, b, code in bl:
        assert int(scales[int(r), int(b)]) == int(code, 16), (r, b, scales[int(r), int(b)])


def test_e2m1_rounding_matches_a_brute_force_nearest_search():
    # every value, every midpoint and its fp32 neighbours, both signs, and
    # values past the largest
    vals = list(E2M1)
    for a, b in zip(E2M1[:-1], E2M1[1:]):
        m = np.float32((a + b) / 2)
        vals += [m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(100))]
    vals += [6.5, 7.0, 1e6, 0.1, 1e-30]
    vals = np.array(vals + [-x for x in vals], np.float32)
    got = e2m1_encode_array(vals)
    for x, c in zip(vals, got):
        d = np.abs(np.abs(np.float64(x)) - E2M1)
        best = np.nonzero(d == d.min())[0]
        want = best[0] if len(best) == 1 else best[best % 2 == 0][0]      # tie -> even code
        want |= 8 if x < 0 else 0
        assert int(c) == int(want), (x, c, want)


@pytest.mark.parametrize("s", [1.0, 3.0, 0.75, 2.0 ** -7])
def test_fp8_static_round_trip_is_exact_on_representable_values(s):
    g = np.random.default_rng(1)
    codes = g.integers(0, 256, size=(8, 40), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x41                                 # no NaN codes
    v = np.array([e4m3_value(c) for c in codes.reshape(-1)]).reshape(codes.shape) * s   # exact in fp32
    q = quantize_fp8_static(v.astype(np.float32), s)
    assert np.array_equal(dequant_fp8_static(q, s), v)


@pytest.mark.parametrize("s", [0.75, 3.0, 0.5])
def test_nvfp4_round_trip_is_exact_on_representable_blocks(s):
    g = np.random.default_rng(2)
    rows, nb = 6, 5
    codes = g.integers(0, 16, size=(rows, nb, 16), dtype=np.uint8)
    codes[:, :, 3] = 7 | (codes[:, :, 3] & 8)                            # each block reaches |6|
    sc = g.integers(0x20, 0x60, size=(rows, nb), dtype=np.uint8)        # normal e4m3 block scales
    blk = np.array([e4m3_value(c) for c in sc.reshape(-1)]).reshape(rows, nb)
    v = E2M1[codes & 7] * np.where(codes & 8, -1.0, 1.0) * blk[:, :, None] * s
    q, qs = quantize_nvfp4_act(v.reshape(rows, nb * 16).astype(np.float32), s)
    assert np.array_equal(qs, sc)
    assert np.array_equal(dequant_nvfp4_act(q, qs, s), v.reshape(rows, nb * 16))


def test_codes_do_not_change_under_a_common_power_of_two():
    g = np.random.default_rng(3)
    v = (g.standard_normal((5, 64)) * np.exp2(g.integers(-4, 4, size=(5, 1)))).astype(np.float32)
    for j in (-6, 5):
        f = np.float32(2.0 ** j)
        assert np.array_equal(quantize_fp8_static(v * f, 1.5 * f), quantize_fp8_static(v, 1.5))
        a, b = quantize_nvfp4_act(v * f, 0.3 * f), quantize_nvfp4_act(v, np.float32(0.3))
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_a_change_stays_inside_its_row_block():
    # NVFP4 blocks are 16 consecutive columns of one row: changing one element
    # can move only the codes of its own block; FP8 codes are per element
    g = np.random.default_rng(4)
    v = g.standard_normal((4, 64)).astype(np.float32)
    c0, s0 = quantize_nvfp4_act(v, 0.2)
    f0 = quantize_fp8_static(v, 0.2)
    for r, c in ((0, 0), (1, 17), (3, 63), (2, 40)):
        w = v.copy()
        w[r, c] = 9.0
        c1, s1 = quantize_nvfp4_act(w, 0.2)
        diff = c0 != c1
        blk = np.zeros_like(diff)
        blk[r, 16 * (c // 16):16 * (c // 16) + 16] = True
        assert not (diff & ~blk).any() and diff[r, c]
        assert (s0 != s1).sum() == 1 and s0[r, c // 16] != s1[r, c // 16]
        f1 = quantize_fp8_static(w, 0.2)
        assert np.array_equal(np.argwhere(f0 != f1), [[r, c]])


# ----------------------------------------------------------------- layers

def _worked_layer(mode):
    rows = {r[1]: [float(x) for x in r[2:]] for r in read_golden("act_quant_layer_worked_example.txt")
            if r[0] == mode}
    if mode == "w4a8":
        H, I = 2, 1
        w13 = np.array([[1.0, 0.0], [0.0, 3.0]])
        w2 = np.array([[1.0], [-2.0]])
        sc, sc2 = [1.0, 2.0], [4.0, 0.5]
    else:
        H, I = 16, 16
        w13 = np.zeros((2 * I, H))
        w13[0, 0] = 1.0
        w13[I, 1] = 1.0
        w2 = np.zeros((H, I))
        w2[0, 0], w2[1, 0] = 1.0, 0.5
        sc, sc2 = [0.25, 0.5], [1.0, 0.75]
    x = np.zeros((2, H))
    x[0, :2], x[1, :2] = rows["x0"], rows["x1"]
    y = np.zeros((2, H))
    y[0, :2], y[1, :2] = rows["y0"], rows["y1"]
    zero = (np.zeros_like(w13), np.zeros_like(w2))
    return x, y, (lambda e: (w13, w2) if e == 0 else zero), sc, sc2


@pytest.mark.parametrize("mode,fn", [("w4a8", moe_layer_w4a8), ("w4a4", moe_layer_w4a4)])
def test_quantising_layers_worked_by_hand(mode, fn):
    x, y_want, weights_of, sc, sc2 = _worked_layer(mode)
    ids = np.zeros((2, 1), np.int64)
    w = np.ones((2, 1))
    y = fn(x, ids, w, weights_of, sc, sc2)
    assert np.array_equal(y, y_want), (y[:, :2], y_want[:, :2])


def _random_layer(seed, T=6, E=4, k=2, H=64, I=32):
    g = np.random.default_rng(seed)
    x = g.standard_normal((T, H)).astype(np.float32).astype(np.float64)
    ws = {e: (g.standard_normal((2 * I, H)) * 0.2, g.standard_normal((H, I)) * 0.2) for e in range(E)}
    ids = np.stack([g.choice(E, k, replace=False) for _ in range(T)])
    w = g.random((T, k))
    return x, ids, w, ws.__getitem__


@pytest.mark.parametrize("fn", [moe_layer_w4a8, moe_layer_w4a4])
def test_layer_depends_on_the_scales_only_through_their_maxima(fn):
    x, ids, w, wf = _random_layer(5)
    y = fn(x, ids, w, wf, [2.0, 3.0, 2.0, 3.0], [1.0, 0.5, 0.5, 0.5])
    assert np.array_equal(y, fn(x, ids, w, wf, [3.0, 0.1, 1.0, 2.9], [0.2, 1.0, 0.0, 0.9]))
    assert not np.array_equal(y, fn(x, ids, w, wf, [2.0, 9.0, 2.0, 3.0], [1.0, 0.5, 0.5, 0.5]))
    assert not np.array_equal(y, fn(x, ids, w, wf, [2.0, 3.0, 2.0, 3.0], [1.0, 0.5, 9.0, 0.5]))
    a1, a2 = layer_activation_scales([2.0, 3.0, 2.0], [0.5, 0.25])
    assert (a1, a2) == (3.0, 0.5)


@pytest.mark.parametrize("fn", [moe_layer_w4a8, moe_layer_w4a4])
def test_a_token_output_depends_on_its_own_input_only(fn):
    x, ids, w, wf = _random_layer(6)
    y = fn(x, ids, w, wf, [1.5] * 4, [0.7] * 4)
    x2 = x.copy()
    x2[2] *= -3.0
    y2 = fn(x2, ids, w, wf, [1.5] * 4, [0.7] * 4)
    assert not np.array_equal(y[2], y2[2])
    keep = np.arange(len(x)) != 2
    assert np.array_equal(y[keep], y2[keep])


@pytest.mark.parametrize("fn", [moe_layer_w4a8, moe_layer_w4a4])
def test_zero_up_projection_gives_the_plain_layer(fn):
    x, ids, w, wf = _random_layer(7)

    def zup(e):
        w13, w2 = wf(e)
        w13 = w13.copy()
        w13[w13.shape[0] // 2:] = 0.0
        return w13, w2
    y = fn(x, ids, w, zup, [1.0] * 4, [1.0] * 4)
    assert np.array_equal(y, moe_layer(x, ids, w, zup)) and not y.any()
