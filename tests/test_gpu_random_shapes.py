"""GPU parity over seeded random layer shapes: token count, expert count, top-k,
hidden and intermediate sizes and weight format drawn per case, so that the
kernel choices (few-rows or wide kernels, four or two activation buffers,
pass slices, split or merged N chunks) meet shapes no hand-picked case covers.
Each case runs the demand path against the oracle (every output element) and
against the whole-layer stream path (bit for bit)."""
import numpy as np
import pytest
import torch

import test_gpu_moe as M
from helpers import flush, rel_max_err

pytestmark = pytest.mark.gpu

N_CASES = 24


def _case(i):
    r = np.random.default_rng(9000 + i)
    wd = ["bf16", "nvfp4", "fp8", "mxfp4"][i % 4]
    E = int(r.choice([2, 3, 8, 12, 16, 40, 64, 128]))
    k = int(r.integers(1, min(E, 8) + 1))
    T = int(r.integers(1, 48)) if r.random() < 0.4 else int(r.integers(1, 700))   # few rows, or many
    H = 128 * int(r.choice([1, 2, 3, 4, 6, 8]))
    I = 128 * int(r.choice([1, 2, 3, 4, 6]))
    return wd, T, E, k, H, I


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_layer_shape_vs_oracle_and_stream(i):
    wd, T, E, k, H, I = _case(i)
    # enough slots for every expert of the layer, queries of up to 16
    s = M._setup(f"random_{i}", S=E + 4, W_=16, wdtype=wd, T=T, E=E, k=k, H=H, I=I, NL=2)
    bank = M._bank_for(s)
    sc = np.ones(E, np.float32)
    d = M._run_demand(s, bank, sc)
    y = M._y(d)
    y_ref, _, _ = M._oracle(s)
    err = rel_max_err(y, y_ref)
    flush(f"random case {i}: {wd} T={T} E={E} k={k} H={H} I={I} m_chunk={d.cfg_used.m_chunk}: "
          f"rel max err = {err:.3e}")
    assert err <= (M.TOL_BF16 if wd == "bf16" else M.TOL_FP4)
    st = M._run_stream(s, sc)
    assert torch.equal(d["y"], st["y"]), "slot path equals the whole-layer path bit for bit"
