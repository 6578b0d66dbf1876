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

W4A8 variant (moe_layer_w4a8): the expert input and the SwiGLU output h are
each quantised to MXFP8 (oracle.lowbit.quantize_mxfp8, per 32 consecutive
columns of a row) before their product with the weights; everything else as
above, in fp64.

Parity: pinned (pure-Python scalar loops on tiny shapes, single-expert
reduction with k = 1, zero up-projection gives zero output; the W4A8 variant
equals the plain layer when every activation and h value is already an MXFP8
value, and its quantiser is pinned in tests/test_oracle_lowbit.py).
"""
import numpy as np

from .lowbit import dequant_mxfp8, quantize_mxfp8


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


def expert_mlp_w4a8(xq: np.ndarray, w13: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """Like expert_mlp on MXFP8 inputs xq [m, H] (already quantised values),
    with h quantised to MXFP8 before the down projection."""
    I = w13.shape[0] // 2
    g = xq @ w13[:I].T
    u = xq @ w13[I:].T
    h = (g / (1.0 + np.exp(-g))) * u
    hq = dequant_mxfp8(*quantize_mxfp8(h))
    return hq @ w2.T


def moe_layer_w4a8(x: np.ndarray, ids: np.ndarray, w: np.ndarray, weights_of) -> np.ndarray:
    """W4A8 routed layer for every token: x [T, H] fp64 is quantised to MXFP8
    per token, each route's h to MXFP8 per route; rank-ordered combine."""
    xq = dequant_mxfp8(*quantize_mxfp8(x))
    T, k = ids.shape
    outs = {}
    by_e = {}
    for t in range(T):
        for j in range(k):
            by_e.setdefault(int(ids[t, j]), []).append((t, j))
    for e, routes in by_e.items():
        w13, w2 = weights_of(e)
        o = expert_mlp_w4a8(np.stack([xq[t] for t, _ in routes]), w13, w2)
        for (t, j), row in zip(routes, o):
            outs[(t, j)] = row
    y = np.zeros_like(x, dtype=np.float64)
    for t in range(T):
        acc = np.zeros(x.shape[1], dtype=np.float64)
        for j in range(k):
            acc = acc + float(w[t, j]) * outs[(t, j)]
        y[t] = acc
    return y
