"""Pins for the NVFP4 decode oracle (CPU)."""
import math

import numpy as np
import torch

from conftest import read_golden
from oracle import dequant_nvfp4, e2m1_value, e4m3_value


def test_e2m1_codes_match_the_ocp_table():
    for code, val in read_golden("e2m1_ocp.txt"):
        v = e2m1_value(int(code))
        assert v == float(val) and math.copysign(1, v) == math.copysign(1, float(val))


def test_e4m3_all_codes_match_torch_float8_e4m3fn():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = np.array([e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert e4m3_value(0x7E) == 448.0 and e4m3_value(0x01) == 2.0 ** -9


def test_nibble_order_block_axis_and_global_scale():
    # row 0: bytes 0x21 -> columns (0, 1) = codes (1, 2) = (0.5, 1.0)
    q = np.zeros((2, 16), np.uint8)
    q[0, 0] = 0x21
    q[1, 15] = 0xF7          # columns 30, 31 = codes (7, 15) = (6, -6)
    s = np.array([[0x38, 0x40], [0x30, 0x48]], np.uint8)   # 1.0, 2.0 / 0.5, 4.0
    w = dequant_nvfp4(q, s, np.float32(0.25))
    assert w.shape == (2, 32)
    assert w[0, 0] == 0.5 * 1.0 * 0.25 and w[0, 1] == 1.0 * 1.0 * 0.25
    assert w[1, 30] == 6.0 * 4.0 * 0.25 and w[1, 31] == -6.0 * 4.0 * 0.25
    assert np.count_nonzero(w) == 4


def test_products_of_codes_are_exact_in_bfloat16():
    # e2m1 * e4m3 has at most 5 significant bits and stays in bf16's range,
    # which is what lets a kernel dequantise to bf16 without rounding
    for q in range(16):
        for s in range(256):
            v = e2m1_value(q) * e4m3_value(s)
            if math.isnan(v):
                continue
            t = torch.tensor(v, dtype=torch.float64)
            assert float(t.to(torch.bfloat16).to(torch.float64)) == v
