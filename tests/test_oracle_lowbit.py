"""Pins for the FP8 and MXFP4 decode oracle (CPU)."""
import math

import numpy as np
import torch

from oracle import dequant_fp8, dequant_mxfp4, e2m1_value, e8m0_value


def test_e8m0_all_codes_match_torch_float8_e8m0fnu():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    mine = np.array([e8m0_value(c) for c in range(256)])
    assert np.isnan(mine[255]) and np.isnan(ref[255])
    assert np.array_equal(mine[:255], ref[:255])
    assert e8m0_value(127) == 1.0 and e8m0_value(0) == 2.0 ** -127 and e8m0_value(254) == 2.0 ** 127


def test_fp8_decode_is_the_e4m3fn_value_times_the_tensor_scale():
    g = np.random.default_rng(5)
    codes = g.integers(0, 256, size=(16, 64), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C            # no NaN codes
    s = np.float32(0.0078125 * 1.25)
    w = dequant_fp8(codes, s)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy() * float(s)
    assert np.array_equal(w, ref)
    assert dequant_fp8(np.array([[0x7E, 0xFE, 0x01]], np.uint8), np.float32(1.0)).tolist() == [[448.0, -448.0, 2.0 ** -9]]


def test_mxfp4_block_axis_nibble_order_and_scaling():
    # row 0: byte 0 = 0x21 -> columns (0, 1) = codes (1, 2) = (0.5, 1.0), block 0 scale 2^1
    # row 1: byte 31 = 0xF7 -> columns (62, 63) = codes (7, 15) = (6, -6), block 1 scale 2^-3
    q = np.zeros((2, 32), np.uint8)
    q[0, 0] = 0x21
    q[1, 31] = 0xF7
    s = np.array([[128, 127], [127, 124]], np.uint8)
    w = dequant_mxfp4(q, s)
    assert w.shape == (2, 64)
    assert w[0, 0] == 0.5 * 2.0 and w[0, 1] == 1.0 * 2.0
    assert w[1, 62] == 6.0 / 8 and w[1, 63] == -6.0 / 8
    assert np.count_nonzero(w) == 4


def test_mxfp4_is_the_e2m1_table_under_unit_scale_and_exact_powers_of_two():
    g = np.random.default_rng(6)
    codes = g.integers(0, 16, size=(4, 64), dtype=np.uint8)
    q = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    table = np.array([e2m1_value(c) for c in range(16)])
    unit = dequant_mxfp4(q, np.full((4, 2), 127, np.uint8))
    assert np.array_equal(unit, table[codes])
    for e in (0, 1, 100, 127, 150, 254):
        w = dequant_mxfp4(q, np.full((4, 2), e, np.uint8))
        assert np.array_equal(w, np.ldexp(table[codes], e - 127))


def test_fp8_and_mxfp4_products_are_exact_in_bfloat16():
    # every finite e4m3 value, and every e2m1 value under E8M0 scale codes
    # 2..252 (which keep every nonzero product in bf16's normal range), is a
    # bf16 value: the kernels decode these formats to bf16 without rounding
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            continue
        v = float(torch.tensor([c], dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64))
        assert float(torch.tensor(v, dtype=torch.float64).to(torch.bfloat16).to(torch.float64)) == v
    for q in range(16):
        for e in range(2, 253):
            v = math.ldexp(e2m1_value(q), e - 127)
            assert v == 0 or abs(v) >= 2.0 ** -126
            assert float(torch.tensor(v, dtype=torch.float64).to(torch.bfloat16).to(torch.float64)) == v


def test_e4m3_encoder_rounds_like_torch_float8_e4m3fn():
    # every code, every midpoint between neighbouring codes and its two fp32
    # neighbours, both signs; torch's conversion is round-to-nearest-even
    from oracle.lowbit import _e4m3_encode_array, e4m3_encode
    pos = torch.arange(0, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    vals = list(pos)
    for a, b in zip(pos[:-1], pos[1:]):
        mid = (a + b) / 2
        vals += [mid, float(np.nextafter(np.float32(mid), np.float32(0))), float(np.nextafter(np.float32(mid), np.float32(1e9)))]
    vals = np.array(vals + [-v for v in vals], dtype=np.float32)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mine = _e4m3_encode_array(vals.astype(np.float64))
    assert np.array_equal(mine, ref)
    assert all(e4m3_encode(float(v)) == int(c) for v, c in zip(vals[::7], ref[::7]))
    assert e4m3_encode(1000.0) == 0x7E and e4m3_encode(-449.0) == 0xFE      # saturation
