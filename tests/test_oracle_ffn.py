"""Pins for the oracle's SwiGLU experts, the grouped FFN and the layer as a
whole (the dense evaluation never touches dispatch or the permutation)."""
import json
import math
import os

import numpy as np
import pytest

from oracle import combine as Cb, dispatch as D, ffn as F, route as R
from moe_inputs import configs as C, generate as gen

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_worked_example():
    g = json.load(open(os.path.join(GOLD, "swiglu_worked.json")))
    ln3 = math.log(3.0)
    w13 = np.array([[ln3 if v == "ln3" else v for v in row] for row in g["w13"]])
    y, flops = F.expert_forward(np.array([g["x"]]), w13, np.array(g["w2"]))
    assert np.allclose(y[0] / ln3, g["y_over_ln3"], rtol=1e-14, atol=0)
    assert flops == g["flops"]


def test_flops_closed_form():
    rng = np.random.default_rng(0)
    d, d_ff, n = 24, 10, 7
    _, flops = F.expert_forward(rng.standard_normal((n, d)), rng.standard_normal((2 * d_ff, d)),
                                rng.standard_normal((d, d_ff)))
    assert flops == n * 6 * d * d_ff


def test_zero_gate_projection_gives_zero():
    rng = np.random.default_rng(1)
    w13 = rng.standard_normal((8, 6))
    w13[:4] = 0.0                       # W1 = 0: silu(0) = 0
    y, _ = F.expert_forward(rng.standard_normal((5, 6)), w13, rng.standard_normal((6, 4)))
    assert np.all(y == 0.0)


def _layer_sparse(x, idx, w, w13, w2, sh13, sh2, E):
    counts, offsets, dest, src = D.dispatch(idx, E)
    xp = D.pack(x, src)
    yp, flops = F.grouped_ffn(xp, offsets, w13, w2)
    ysh, fsh = F.expert_forward(x, sh13, sh2)
    return Cb.combine(yp, dest, w, ysh=ysh), flops + fsh


def _layer_dense(x, idx, w, w13, w2, sh13, sh2, E):
    T = x.shape[0]
    gate = np.zeros((T, E))
    np.put_along_axis(gate, idx.astype(np.int64), w.astype(np.float64), axis=1)
    out, _ = F.expert_forward(x, sh13, sh2)
    for e in range(E):
        ye, _ = F.expert_forward(x, w13[e], w2[e])
        out = out + gate[:, e:e + 1] * ye
    return out


@pytest.mark.parametrize("name,T", [("tiny", 256), ("flash", 48)])
def test_dense_equals_sparse(name, T):
    cfg = C.get(name).with_(T=T)
    if name == "flash":
        cfg = cfg.with_(d=256, d_ff=128)     # keep the CPU time small; same routing shape
    inp = gen.make_router(cfg)
    ex = gen.make_experts(cfg)
    x = inp["x"].float().numpy()
    L, idx, w = R.route(x, inp["w_gate"].numpy(), inp["bias"].numpy(), cfg.G, cfg.M, cfg.k, cfg.gk)
    args = (x, idx, w, ex["w13"].float().numpy(), ex["w2"].float().numpy(),
            ex["sh_w13"][0].float().numpy(), ex["sh_w2"][0].float().numpy(), cfg.E)
    sparse, flops = _layer_sparse(*args)
    dense = _layer_dense(*args)
    assert np.allclose(sparse, dense, rtol=1e-12, atol=1e-12 * np.abs(dense).max())
    assert flops == (T * cfg.k + T) * 6 * cfg.d * cfg.d_ff


def test_hidden_worked_example():
    # expert_hidden feeds the fp8 emulation: h = silu(x W1^T) * (x W3^T) = 1.5 ln3
    # on the hand-derived example (a W1/W3 swap gives 2 sigmoid(2) ln3 instead)
    g = json.load(open(os.path.join(GOLD, "swiglu_worked.json")))
    ln3 = math.log(3.0)
    w13 = np.array([[ln3 if v == "ln3" else v for v in row] for row in g["w13"]])
    h = F.expert_hidden(np.array([g["x"]]), w13)
    assert h.shape == (1, 1)
    assert abs(h[0, 0] - 1.5 * ln3) <= 1e-15 * ln3


def test_hidden_then_down_projection_is_the_expert():
    # h W2^T of expert_hidden equals expert_forward on random rows, and a swap
    # of the gate and up halves of w13 changes the result
    rng = np.random.default_rng(5)
    d, d_ff, n = 16, 12, 9
    X = rng.standard_normal((n, d))
    w13 = rng.standard_normal((2 * d_ff, d))
    w2 = rng.standard_normal((d, d_ff))
    y, _ = F.expert_forward(X, w13, w2)
    h = F.expert_hidden(X, w13)
    assert h.shape == (n, d_ff)
    assert np.allclose(h @ w2.T, y, rtol=1e-13, atol=1e-13 * np.abs(y).max())
    swapped = np.concatenate([w13[d_ff:], w13[:d_ff]])
    assert not np.allclose(F.expert_hidden(X, swapped), h)
