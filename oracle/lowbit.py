"""FP8 and MXFP4 weight decode (oracle).

Source: FreeToken PR #676, "Known limits": besides NVFP4, the prefill over the
slots also runs bf16, FP8 and MXFP4 expert weights.  The pages name the
formats and nothing more, so their encodings are taken from the OCP
Microscaling Formats specification:

* FP8 here is OCP FP8 E4M3 (the "FN" variant: no infinities, one NaN pattern
  per sign), one byte per weight, with one fp32 scale per (expert, tensor)
  that multiplies the decoded byte, as the NVFP4 global scale does.  A
  per-tensor scale is the plainest reading of "FP8 weights"; per-row or
  per-block scales are not described on the pages.
* MXFP4 is the MX format with FP4 E2M1 elements and one E8M0 scale per block
  of 32 consecutive elements: value = e2m1(code) * 2^(scale - 127), the scale
  code 255 being NaN.  As for NVFP4, the block runs along the input (K)
  dimension of each weight row and the low nibble of a byte is the even
  column.  MX has no second-level scale.

Everything is formed in fp64, exactly.

Parity: pinned (E8M0 for all 256 codes against torch.float8_e8m0fnu, the E4M3
decode already pinned for NVFP4 scales, the block axis and nibble order by a
hand-worked example, the MX scaling law by its closed form).
"""
import numpy as np

from .nvfp4 import e2m1_value, e4m3_value


def e8m0_value(code: int) -> float:
    """Value of an 8-bit E8M0 scale code: 2^(code - 127); 255 is NaN."""
    code = int(code) & 0xFF
    if code == 0xFF:
        return float("nan")
    return 2.0 ** (code - 127)


_E2M1_LUT = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
_E4M3_LUT = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
_E8M0_LUT = np.array([e8m0_value(c) for c in range(256)], dtype=np.float64)


def dequant_fp8(codes: np.ndarray, g) -> np.ndarray:
    """Decode one FP8 (E4M3FN) tensor: W[r, c] = e4m3(codes[r, c]) * g, fp64.

    codes uint8 [rows, cols], g float32 (the tensor's scale)."""
    return _E4M3_LUT[np.asarray(codes, dtype=np.uint8)] * float(np.float32(g))


def dequant_mxfp4(q_packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Decode one MXFP4 tensor to fp64.

    q_packed uint8 [rows, cols/2] (low nibble = even column), scales uint8
    [rows, cols/32] (E8M0).  W[r, c] = e2m1(q[r, c]) * 2^(s[r, c // 32] - 127)."""
    q = np.asarray(q_packed, dtype=np.uint8)
    rows, half = q.shape
    cols = half * 2
    codes = np.empty((rows, cols), dtype=np.uint8)
    codes[:, 0::2] = q & 0xF
    codes[:, 1::2] = q >> 4
    s = _E8M0_LUT[np.asarray(scales, dtype=np.uint8)]
    s_full = np.repeat(s, 32, axis=1)
    assert s_full.shape == (rows, cols)
    return _E2M1_LUT[codes] * s_full


# ---------------------------------------------------------------- E4M3 encode
# Nearest E4M3FN code to a value, ties to the even code, magnitudes beyond the
# format saturated to 448 (used by the activation quantisers, oracle/actquant.py).

_E4M3_POS = np.array([e4m3_value(c) for c in range(0x7F)], dtype=np.float64)   # codes 0x00..0x7E, ascending


def e4m3_encode(v: float) -> int:
    """Nearest e4m3 code to a finite value, ties to the even code, |v| > 448
    saturated to 448."""
    v = float(v)
    sign = 0x80 if (v < 0 or (v == 0 and np.signbit(v))) else 0
    a = min(abs(v), 448.0)
    i = int(np.searchsorted(_E4M3_POS, a))          # first code with value >= a
    if i < len(_E4M3_POS) and _E4M3_POS[i] == a:
        return sign | i
    lo, hi = i - 1, i                                # a lies strictly between codes lo and hi
    dlo, dhi = a - _E4M3_POS[lo], _E4M3_POS[hi] - a
    c = lo if (dlo < dhi or (dlo == dhi and lo % 2 == 0)) else hi
    return sign | c


def _e4m3_encode_array(a: np.ndarray) -> np.ndarray:
    """e4m3_encode over an array (the same rule, vectorised)."""
    a = np.asarray(a, dtype=np.float64)
    sign = np.where(np.signbit(a), 0x80, 0).astype(np.uint8)
    m = np.minimum(np.abs(a), 448.0)
    hi = np.minimum(np.searchsorted(_E4M3_POS, m), len(_E4M3_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = m - _E4M3_POS[lo], _E4M3_POS[hi] - m
    exact = _E4M3_POS[hi] == m
    pick_lo = (dlo < dhi) | ((dlo == dhi) & (lo % 2 == 0))
    code = np.where(exact, hi, np.where(pick_lo, lo, hi)).astype(np.uint8)
    return sign | code
