"""Pins for the oracle's combine."""
import numpy as np

from oracle import combine as Cb, dispatch as D


def _route(rng, T, E, k):
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k))
    return idx, w / w.sum(1, keepdims=True)


def test_identity_experts_return_weight_sum_times_x():
    rng = np.random.default_rng(0)
    T, E, k, d = 300, 16, 4, 12
    idx, w = _route(rng, T, E, k)
    w = w * rng.random((T, 1)) * 3       # arbitrary weight sums
    x = rng.standard_normal((T, d))
    _, _, dest, src = D.dispatch(idx, E)
    yp = D.pack(x, src)                  # identity expert: y = x
    out = Cb.combine(yp, dest, w)
    assert np.allclose(out, w.sum(1, keepdims=True) * x, rtol=1e-13, atol=1e-13)


def test_one_hot_gate_is_a_gather():
    rng = np.random.default_rng(1)
    T, E, k, d = 100, 8, 3, 5
    idx, _ = _route(rng, T, E, k)
    w = np.zeros((T, k))
    w[:, 1] = 1.0
    _, _, dest, _ = D.dispatch(idx, E)
    yp = rng.standard_normal((T * k, d))
    out = Cb.combine(yp, dest, w)
    assert np.array_equal(out, yp[dest[:, 1]])


def test_shared_term_and_accumulate():
    rng = np.random.default_rng(2)
    T, E, k, d = 64, 8, 2, 4
    idx, w = _route(rng, T, E, k)
    _, _, dest, _ = D.dispatch(idx, E)
    yp = rng.standard_normal((T * k, d))
    ysh = rng.standard_normal((T, d))
    base = Cb.combine(yp, dest, w)
    assert np.allclose(Cb.combine(yp, dest, w, ysh=ysh), base + ysh)
    init = rng.standard_normal((T, d))
    assert np.allclose(Cb.combine(yp, dest, w, out_init=init), base + init)


def test_nonlocal_slots_skipped():
    rng = np.random.default_rng(3)
    T, E, k, d = 80, 16, 4, 3
    idx, w = _route(rng, T, E, k)
    c, o, dest, src = D.dispatch(idx, E, 0, 4)
    yp = rng.standard_normal((int(o[-1]), d))
    out = Cb.combine(yp, dest, w)
    ref = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            if idx[t, j] < 4:
                ref[t] += w[t, j] * yp[dest[t, j]]
    assert np.allclose(out, ref)
