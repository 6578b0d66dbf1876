"""Pins for the expert-MLP / combine oracle (CPU)."""
import math

import numpy as np

from oracle import expert_mlp, moe_layer
from oracle.mlp import bf16_bits_to_f64


def _scalar_layer(x, ids, w, experts):
    """Pure-Python scalar loops, independent of numpy's matmul."""
    T, H = len(x), len(x[0])
    k = len(ids[0])
    y = [[0.0] * H for _ in range(T)]
    for t in range(T):
        for j in range(k):
            w13, w2 = experts[ids[t][j]]
            I = len(w13) // 2
            h = []
            for i in range(I):
                g = sum(w13[i][c] * x[t][c] for c in range(H))
                u = sum(w13[I + i][c] * x[t][c] for c in range(H))
                h.append(g / (1.0 + math.exp(-g)) * u)
            for c in range(H):
                y[t][c] += w[t][j] * sum(w2[c][i] * h[i] for i in range(I))
    return y


def _tiny(seed=3, T=4, H=5, I=3, E=3, k=2):
    g = np.random.default_rng(seed)
    x = g.standard_normal((T, H))
    experts = {e: (g.standard_normal((2 * I, H)), g.standard_normal((H, I))) for e in range(E)}
    ids = np.array([g.choice(E, size=k, replace=False) for _ in range(T)])
    w = g.random((T, k)).astype(np.float32)
    return x, ids, w, experts


def test_matches_scalar_loops_on_a_tiny_layer():
    x, ids, w, experts = _tiny()
    y = moe_layer(x, ids, w, lambda e: experts[e])
    ref = _scalar_layer(x.tolist(), ids.tolist(), w.astype(np.float64).tolist(),
                        {e: (a.tolist(), b.tolist()) for e, (a, b) in experts.items()})
    assert np.allclose(y, np.array(ref), rtol=1e-12, atol=1e-12)


def test_k1_unit_weight_is_one_expert_mlp():
    x, _, _, experts = _tiny(T=6)
    ids = np.array([[2]] * 6)
    w = np.ones((6, 1), np.float32)
    y = moe_layer(x, ids, w, lambda e: experts[e])
    assert np.array_equal(y, expert_mlp(x, *experts[2]))


def test_zero_up_projection_gives_zero_output():
    x, ids, w, experts = _tiny()
    z = {e: (np.concatenate([a[:3], np.zeros_like(a[3:])]), b) for e, (a, b) in experts.items()}
    assert np.all(moe_layer(x, ids, w, lambda e: z[e]) == 0.0)


def test_bf16_bits_decode():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x7F7F], np.uint16)
    v = bf16_bits_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -1.0 and v[3] == 0.0
    assert v[2] == 3.140625 and v[4] == float.fromhex("0x1.fep127")
