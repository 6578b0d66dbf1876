"""SwiGLU expert MLP and weighted top-k combine (oracle), fp64.

Sources: FreeToken PR #676, "Solution" (the demand chunk runs the same
grouped GEMM over its layer's slot pool at their slots as the streamed
layer) and the workloads' definition of the experts as SwiGLU MLPs whose
outputs are combined with the routing weights.

Definition:  y[t] = sum_j w[t, j] * W2_e (silu(G_e x_t) * (U_e x_t)),  e = ids[t, j],
where G_e = W13_e[0:I], U_e = W13_e[I:2I] (w13 is [2I, H], gate rows first),
W2_e is [H, I] and silu(z) = z / (1 + exp(-z)).  The sum over j runs in rank
order.  Inputs are the exact values the device receives (bf16 or decoded
NVFP4), widened to fp64; nothing is rounded on the way.

Activation-quantising variants (FreeToken PR #676, Solution, fourth bullet:
the W4A4 GEMM quantises its activations under the max of the routed layer's
input scales): ``moe_layer_w4a8`` and ``moe_layer_w4a4`` quantise x (per
token) under the max of the layer's gate/up input scales and each route's h
(per route, after SwiGLU) under the max of its down input scales, with the
rules of oracle/actquant.py (FP8 E4M3 per tensor for W4A8, NVFP4 with the
layer scale as global scale for W4A4), then continue in fp64 as above.

Parity: pinned (pure-Python scalar loops on tiny shapes, single-expert
reduction with k = 1, zero up-projection gives zero output).  The quantising
variants by: a hand-worked two-token layer (tests/golden/
act_quant_layer_worked_example.txt), equality with the plain layer when x is
representable and the up projection is zero, dependence on the input scales
only through their maxima, token locality (y[t] depends on x[t] alone), and
the quantisers' own pins.
"""
import numpy as np

from .actquant import (dequant_fp8_static, dequant_nvfp4_act, layer_activation_scales, quantize_fp8_static,
                       quantize_nvfp4_act)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64 values."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def expert_mlp(x: np.ndarray, w13: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """x [m, H] fp64, w13 [2I, H], w2 [H, I] -> [m, H]: W2 (silu(G x) * (U x)) per row."""
    I = w13.shape[0] // 2
    g = x @ w13[:I].T
    u = x @ w13[I:].T
    h = (g / (1.0 + np.exp(-g))) * u
    return h @ w2.T


def moe_layer_tokens(x: np.ndarray, ids: np.ndarray, w: np.ndarray, weights_of, tokens) -> np.ndarray:
    """Routed layer output for the listed tokens only.

    x [T, H] fp64, ids int [T, k], w float [T, k], weights_of(e) -> (w13, w2)
    in fp64.  Returns fp64 [len(tokens), H].
    """
    tokens = np.asarray(list(tokens), dtype=np.int64)
    k = ids.shape[1]
    H = x.shape[1]
    # every (token, rank) route's expert output, evaluated expert by expert so
    # each expert's weights are widened once; values do not depend on grouping
    outs = {}
    by_e = {}
    for t in tokens:
        for j in range(k):
            by_e.setdefault(int(ids[t, j]), []).append((int(t), j))
    for e, routes in by_e.items():
        w13, w2 = weights_of(e)
        xs = np.stack([x[t] for t, _ in routes])
        o = expert_mlp(xs, w13, w2)
        for (t, j), row in zip(routes, o):
            outs[(t, j)] = row
    y = np.zeros((tokens.size, H), dtype=np.float64)
    for i, t in enumerate(tokens):
        acc = np.zeros(H, dtype=np.float64)
        for j in range(k):                      # rank order
            acc = acc + float(w[t, j]) * outs[(int(t), j)]
        y[i] = acc
    return y


def moe_layer(x, ids, w, weights_of):
    """Routed layer output for every token: fp64 [T, H]."""
    return moe_layer_tokens(x, ids, w, weights_of, range(x.shape[0]))


def _quantised(mode: str, v: np.ndarray, scale) -> np.ndarray:
    """The values the GEMM sees for activations v [rows, cols] under a layer scale."""
    if mode == "w4a8":
        return dequant_fp8_static(quantize_fp8_static(v, scale), scale)
    if mode == "w4a4":
        return dequant_nvfp4_act(*quantize_nvfp4_act(v, scale), scale)
    raise ValueError(mode)


def moe_layer_act_quant(mode: str, x: np.ndarray, ids: np.ndarray, w: np.ndarray, weights_of, input_scale,
                        down_input_scale) -> np.ndarray:
    """Routed layer with quantised activations, every token: fp64 [T, H].

    x [T, H] (the bf16 values, as fp64) is quantised per token under
    a1 = max(input_scale); each route's h = silu(G xq) * (U xq), in fp64, is
    quantised per route under a2 = max(down_input_scale); o = W2 hq; y[t] is
    the rank-ordered sum of w[t, j] * o over the token's routes."""
    a1, a2 = layer_activation_scales(input_scale, down_input_scale)
    xq = _quantised(mode, x, a1)
    T, k = ids.shape
    I = None
    outs = {}
    by_e = {}
    for t in range(T):
        for j in range(k):
            by_e.setdefault(int(ids[t, j]), []).append((t, j))
    for e, routes in by_e.items():
        w13, w2 = weights_of(e)
        I = w13.shape[0] // 2
        xs = np.stack([xq[t] for t, _ in routes])
        g = xs @ w13[:I].T
        u = xs @ w13[I:].T
        h = (g / (1.0 + np.exp(-g))) * u                  # one row per route
        o = _quantised(mode, h, a2) @ w2.T
        for (t, j), row in zip(routes, o):
            outs[(t, j)] = row
    y = np.zeros_like(x, dtype=np.float64)
    for t in range(T):
        acc = np.zeros(x.shape[1], dtype=np.float64)
        for j in range(k):                                 # rank order
            acc = acc + float(w[t, j]) * outs[(t, j)]
        y[t] = acc
    return y


def moe_layer_w4a8(x, ids, w, weights_of, input_scale, down_input_scale):
    """W4A8: FP8 E4M3 activations (one scale per tensor) under the layer's scales."""
    return moe_layer_act_quant("w4a8", x, ids, w, weights_of, input_scale, down_input_scale)


def moe_layer_w4a4(x, ids, w, weights_of, input_scale, down_input_scale):
    """W4A4: NVFP4 activations with the layer's scales as their global scales."""
    return moe_layer_act_quant("w4a4", x, ids, w, weights_of, input_scale, down_input_scale)
