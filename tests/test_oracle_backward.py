"""Pins for the oracle's layer backward: every gradient against torch.autograd
(fp64, CPU) over the same forward with the expert selection held fixed, plus a
finite-difference check of the gate path."""
import numpy as np
import pytest
import torch

from oracle import backward as B
from oracle import combine as OC, dispatch as OD, ffn as OF, route as OR


def _setup(seed=0, T=40, d=24, E=8, G=4, M=2, k=3, d_ff=16):
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(T, d))
    wg = rng.normal(size=(d, E)) * 0.3
    bias = rng.uniform(-0.1, 0.1, size=E).astype(np.float32)
    w13 = rng.normal(size=(E, 2 * d_ff, d)) * 0.2
    w2 = rng.normal(size=(E, d, d_ff)) * 0.2
    s13 = rng.normal(size=(2 * d_ff, d)) * 0.2
    s2 = rng.normal(size=(d, d_ff)) * 0.2
    g = rng.normal(size=(T, d))
    L64 = x @ wg
    idx, _ = OR.route_from_logits(L64.astype(np.float32), bias, G, M, k, -(-k // M))
    # the selection comes from the fp32 logits; derivatives are taken at the
    # fp64 logits, as torch does
    return dict(x=x, wg=wg, w13=w13, w2=w2, s13=s13, s2=s2, g=g, L=L64, idx=idx, E=E, d_ff=d_ff)


def _torch_grads(p):
    t = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    x, wg, w13, w2, s13, s2 = (t(p[n]) for n in ("x", "wg", "w13", "w2", "s13", "s2"))
    idx = torch.tensor(p["idx"], dtype=torch.long)
    d_ff = p["d_ff"]

    def expert(X, a13, a2):
        a = X @ a13[:d_ff].T
        u = X @ a13[d_ff:].T
        return (torch.nn.functional.silu(a) * u) @ a2.T

    L = x @ wg
    s = torch.sqrt(torch.nn.functional.softplus(L))
    sel = torch.gather(s, 1, idx)
    w = sel / sel.sum(1, keepdim=True)
    out = expert(x, s13, s2)
    T, k = idx.shape
    rows = []
    for tt in range(T):
        acc = 0
        for j in range(k):
            e = int(idx[tt, j])
            acc = acc + w[tt, j] * expert(x[tt:tt + 1], w13[e], w2[e])[0]
        rows.append(acc)
    out = out + torch.stack(rows)
    out.backward(torch.tensor(p["g"], dtype=torch.float64))
    return {n: v.grad.numpy() for n, v in (("x", x), ("wg", wg), ("w13", w13), ("w2", w2),
                                            ("s13", s13), ("s2", s2))}


def _oracle_grads(p):
    x, g, idx = p["x"], p["g"], p["idx"]
    T = x.shape[0]
    counts, offsets, dest, src = OD.dispatch(idx, p["E"])
    xp = OD.pack(x, src)
    yp, _ = OF.grouped_ffn(xp, offsets, p["w13"], p["w2"])
    s = np.sqrt(np.logaddexp(0.0, p["L"]))
    sel = np.take_along_axis(s, idx.astype(np.int64), 1)
    w = sel / sel.sum(1, keepdims=True)
    d_yp, d_w = B.combine_backward(g, yp, dest, w, int(offsets[-1]))
    d_xp, dW13, dW2 = B.grouped_ffn_backward(xp, offsets, p["w13"], p["w2"], d_yp)
    dx = B.dispatch_backward(d_xp, dest, T)
    dxs, dS13, dS2 = B.expert_backward(x, p["s13"], p["s2"], g)
    dxg, dWg, dL = B.gate_backward(x, p["wg"], p["L"], idx, d_w)
    return {"x": dx + dxs + dxg, "wg": dWg, "w13": dW13, "w2": dW2, "s13": dS13, "s2": dS2}


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_gradients_match_torch_autograd(seed):
    p = _setup(seed)
    ref = _torch_grads(p)
    got = _oracle_grads(p)
    for n in ref:
        err = np.abs(got[n] - ref[n]).max() / max(np.abs(ref[n]).max(), 1e-300)
        assert err < 1e-10, (n, err)


def test_gate_path_finite_differences():
    # loss(L) = sum_j c_j w_j(L) with the selection fixed: dL from gate_backward
    # against central differences of the renormalised sqrt-softplus weights
    rng = np.random.default_rng(5)
    T, E, k = 6, 8, 3
    L = rng.normal(size=(T, E)) * 2
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    c = rng.normal(size=(T, k))
    x = np.eye(T, 4)
    wg = np.zeros((4, E))
    _, _, dL = B.gate_backward(x, wg, L, idx, c)

    def loss(Lm):
        s = np.sqrt(np.logaddexp(0.0, Lm))
        sel = np.take_along_axis(s, idx.astype(np.int64), 1)
        return float((c * sel / sel.sum(1, keepdims=True)).sum())

    h = 1e-6
    for t in range(T):
        for e in range(E):
            Lp, Lm = L.copy(), L.copy()
            Lp[t, e] += h
            Lm[t, e] -= h
            fd = (loss(Lp) - loss(Lm)) / (2 * h)
            assert abs(fd - dL[t, e]) < 1e-7, (t, e, fd, dL[t, e])


def test_unrouted_slots_get_no_gradient():
    dest = np.array([[0, -1], [1, 2]])
    w = np.array([[0.5, 0.5], [0.25, 0.75]])
    g = np.ones((2, 3))
    yp = np.arange(9.0).reshape(3, 3)
    d_yp, d_w = B.combine_backward(g, yp, dest, w, 3)
    assert d_w[0, 1] == 0.0 and d_w[0, 0] == yp[0].sum()
    assert np.allclose(d_yp[2], 0.75) and np.allclose(d_yp[0], 0.5)
    dx = B.dispatch_backward(np.ones((3, 3)), dest, 2)
    assert dx[0].tolist() == [1.0] * 3 and dx[1].tolist() == [2.0] * 3
