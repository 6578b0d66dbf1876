"""Activation quantisation under the routed layer's input scales (oracle).

Source: FreeToken PR #676, Solution (fourth bullet) and Tests (fourth
bullet): the W4A4 prefill quantises its activations under the largest of the
input scales, and over the slot cache it must take the routed layer's scales
(there 2.0 and 3.0), never the scales of whatever else sits in the slots
(9.0).  The pages name the rule and not the encodings, so:

* ``layer_activation_scales``: the scale of a GEMM's input is the maximum of
  the routed layer's per-expert input scales for that GEMM.  A layer carries
  one array for the gate/up input x and one for the down input h (each
  quantised linear layer of a checkpoint has its own input scale; reading).
* W4A8 (``quantize_fp8_static``): FP8 E4M3 codes of v times the reciprocal
  of the scale, one scale per tensor, rounded to nearest even and saturated
  to +-448 (the static FP8 activation scheme).  Decoded value = e4m3(code) *
  scale.
* W4A4 (``quantize_nvfp4_act``): NVFP4 activations with the layer scale as
  the second-level (global) scale: per 16 consecutive columns of a row the
  block scale is the e4m3 code of amax / (6 * scale) (6 = the largest e2m1
  value), and each element the e2m1 code of v times the reciprocal of
  (block * scale); decoded value = e2m1(code) * e4m3(block) * scale.  A
  block whose scale rounds to zero gets zero codes.

Where these decisions are made in floating point (a quotient or a product,
then a rounding to a code), they are made in fp32, the precision the kernels
use: v and the scale are fp32 values; 6 * scale and block * scale are fp32
products; amax / (6 * scale) is an IEEE fp32 division; the reciprocals 1 /
scale (once per tensor) and 1 / (block * scale) (once per block) are IEEE
fp32 divisions, and each element is multiplied by its reciprocal in fp32 (a
quantiser multiplies by the inverse scale rather than dividing every
element).  The roundings to codes are exact operations on those fp32 values.
Everything after the codes (decoding, the GEMMs) is fp64.

e2m1 rounding: to the nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6 with ties to the
even code (0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4,
5 -> 4), magnitudes above 6 saturated to 6; the sign bit is set for every
negative input, including one that rounds to zero.

Parity: pinned (tests/test_oracle_actquant.py): hand-worked codes in
tests/golden/act_quant_worked_example.txt, the e2m1 rounding against a brute
force nearest-value search with every tie, the e4m3 rounding against
torch.float8_e4m3fn (tests/test_oracle_lowbit.py), exact round trips on
representable inputs, invariance of the codes under a common power-of-two
scaling, block locality along each row, and the layer-level properties in
oracle/mlp.py's pins.
"""
import numpy as np

from .lowbit import _e4m3_encode_array
from .nvfp4 import e2m1_value, e4m3_value

_E2M1_LUT = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
_E4M3_LUT = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def layer_activation_scales(input_scale, down_input_scale):
    """(scale of x, scale of h): the maxima of the layer's two arrays of
    per-expert input scales, as fp32 values."""
    a1 = np.float32(np.max(np.asarray(input_scale, dtype=np.float32)))
    a2 = np.float32(np.max(np.asarray(down_input_scale, dtype=np.float32)))
    return a1, a2


# ----------------------------------------------------------------- W4A8

def quantize_fp8_static(v: np.ndarray, scale) -> np.ndarray:
    """E4M3 codes (uint8, same shape) of fp32(v) * fp32(1 / fp32(scale))."""
    q = np.asarray(v, dtype=np.float32) * (np.float32(1.0) / np.float32(scale))
    return _e4m3_encode_array(q.astype(np.float64)).reshape(np.shape(v))


def dequant_fp8_static(codes: np.ndarray, scale) -> np.ndarray:
    """e4m3(code) * scale in fp64."""
    return _E4M3_LUT[np.asarray(codes, dtype=np.uint8)] * float(np.float32(scale))


# ----------------------------------------------------------------- W4A4

def e2m1_encode_array(q: np.ndarray) -> np.ndarray:
    """e2m1 codes (uint8, 0..15) of fp32 values: nearest, ties to even, |q| > 6 -> 6."""
    q = np.asarray(q, dtype=np.float32)
    m = np.abs(q)
    mag = ((m > 0.25).astype(np.uint8) + (m >= 0.75) + (m > 1.25) + (m >= 1.75) + (m > 2.5) + (m >= 3.5)
           + (m > 5.0)).astype(np.uint8)
    return (mag | np.where(q < 0, 8, 0).astype(np.uint8)).astype(np.uint8)


def quantize_nvfp4_act(v: np.ndarray, scale):
    """NVFP4 codes of a [rows, cols] array (cols a multiple of 16) under the
    global scale: (codes uint8 [rows, cols] one code per element, block
    scale codes uint8 [rows, cols / 16])."""
    v = np.asarray(v, dtype=np.float32)
    rows, cols = v.shape
    s = np.float32(scale)
    blocks = v.reshape(rows, cols // 16, 16)
    amax = np.max(np.abs(blocks), axis=2)                                   # exact in fp32
    d = amax / (np.float32(6.0) * s)                                        # fp32 product, fp32 quotient
    sc = _e4m3_encode_array(d.astype(np.float64)).astype(np.uint8)          # saturates at 448
    sv = _E4M3_LUT[sc].astype(np.float32)                                   # exact in fp32
    den = sv * s                                                            # fp32 product
    live = (sv > 0)[:, :, None]
    rcp = np.float32(1.0) / np.where(live, den[:, :, None], np.float32(1.0))  # fp32 reciprocal per block
    q = blocks * rcp                                                        # fp32 products
    codes = e2m1_encode_array(q)
    # a zero block scale keeps only the signs (every element rounds to zero)
    codes = np.where(live, codes, np.where(blocks < 0, 8, 0)).astype(np.uint8)
    return codes.reshape(rows, cols), sc


def dequant_nvfp4_act(codes: np.ndarray, scales: np.ndarray, scale) -> np.ndarray:
    """e2m1(code) * e4m3(block scale) * scale in fp64, [rows, cols]."""
    c = np.asarray(codes, dtype=np.uint8)
    rows, cols = c.shape
    b = np.repeat(_E4M3_LUT[np.asarray(scales, dtype=np.uint8)], 16, axis=1)
    return _E2M1_LUT[c] * b * float(np.float32(scale))
