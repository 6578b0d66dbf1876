"""NVFP4 weight decode (oracle).

Source: the long-prefill workload's weight format (FP4 e2m1 values, one e4m3
scale per 16-element block, one fp32 global scale per tensor), as NVFP4 is
named for the pool's expert rows in vLLM fork PR #48 ("What": NVFP4 weights
and block scales in pinned host memory) and FreeToken PR #676 ("Solution":
the NVFP4 prefill).  The encodings themselves are the OCP Microscaling
Formats specification's FP4 E2M1 and FP8 E4M3 (the "FN" variant: no
infinities, one NaN pattern per sign).

Readings taken: the 16-element block runs along the input (K) dimension of
each weight row; a byte holds two codes, the low nibble being the even
column; the decoded weight is e2m1 * e4m3 * global, in that order of
meaning (the product is formed in fp64 here, exactly).

Parity: pinned (all 256 e4m3 codes against torch.float8_e4m3fn, the 16 e2m1
codes against the OCP table in tests/golden, torch.float4_e2m1fn_x2 unpacking).
"""
import numpy as np


def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code: sign | 2-bit exponent (bias 1) | 1-bit mantissa."""
    code = int(code) & 0xF
    sign = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        mag = m * 0.5                      # subnormal: 0.m * 2^(1-1)
    else:
        mag = (1.0 + m * 0.5) * 2.0 ** (e - 1)
    return sign * mag


def e4m3_value(code: int) -> float:
    """Value of an 8-bit E4M3FN code: sign | 4-bit exponent (bias 7) | 3-bit mantissa."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        mag = (m / 8.0) * 2.0 ** -6
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return sign * mag


_E2M1_LUT = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
_E4M3_LUT = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def dequant_nvfp4(q_packed: np.ndarray, scales: np.ndarray, g) -> np.ndarray:
    """Decode one NVFP4 tensor to fp64.

    q_packed uint8 [rows, cols/2], scales uint8 [rows, cols/16], g float32.
    Returns float64 [rows, cols] with W[r, c] = e2m1(q[r, c]) * e4m3(s[r, c // 16]) * g.
    """
    q = np.asarray(q_packed, dtype=np.uint8)
    rows, half = q.shape
    cols = half * 2
    codes = np.empty((rows, cols), dtype=np.uint8)
    codes[:, 0::2] = q & 0xF
    codes[:, 1::2] = q >> 4
    s = _E4M3_LUT[np.asarray(scales, dtype=np.uint8)]
    s_full = np.repeat(s, 16, axis=1)
    assert s_full.shape == (rows, cols)
    return _E2M1_LUT[codes] * s_full * float(np.float32(g))
