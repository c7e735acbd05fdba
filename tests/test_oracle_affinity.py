"""Pins for the oracle's fp32 affinity sqrt(softplus(l)).

The fp32 evaluation is an approximation; it is pinned against fp64 libm
(np.logaddexp, np.sqrt in float64) and against values fixed by mathematics.
"""
import numpy as np
import pytest

from oracle import affinity as A


def _ulps(got, ref64):
    ref32 = ref64.astype(np.float32)
    return np.abs(got.astype(np.float64) - ref64) / np.spacing(np.abs(ref32)).astype(np.float64)


def _sweep(stride=97):
    pos = np.arange(0, np.float32(88.0).view(np.uint32), stride, dtype=np.uint32).view(np.float32)
    neg = -np.arange(0, np.float32(86.9).view(np.uint32), stride, dtype=np.uint32).view(np.float32)
    return np.concatenate([pos, neg])


def test_accuracy_dense_sweep():
    l = _sweep()
    s = A.affinity(l)
    ref = np.sqrt(np.logaddexp(0.0, l.astype(np.float64)))
    err = _ulps(s, ref)
    assert err.max() <= 4.0, (err.max(), l[err.argmax()])


@pytest.mark.parametrize("start", [0.0, -1.0e-30, 1.0e-3, -1.0e-3, 0.5, -0.5, 1.0, -1.7, 3.0, -9.0, 20.0, -40.0])
def test_accuracy_consecutive_window(start):
    # every representable fp32 in a window of 2^18 values next to `start`
    b = np.float32(start).view(np.uint32)
    l = (b + np.arange(1 << 18, dtype=np.uint32)).view(np.float32)
    l = l[np.isfinite(l) & (np.abs(l) < 86.9)]
    s = A.affinity(l)
    ref = np.sqrt(np.logaddexp(0.0, l.astype(np.float64)))
    assert _ulps(s, ref).max() <= 4.0


def test_monotone_within_three_ulp():
    # The exact function is increasing; an fp32 evaluation that is not
    # correctly rounded can step back by a few ulp where s changes by less
    # than an ulp between neighbouring inputs (near l = 0 it moves ~1/3 ulp
    # per input ulp).  Both sides use the same operation sequence, so such
    # near-ties are decided identically on the GPU and here.
    l = np.sort(_sweep(stride=31))
    s = A.affinity(l).astype(np.float64)
    drop = s[:-1] - s[1:]
    assert np.all(drop <= 3 * np.spacing(s[:-1].astype(np.float32)).astype(np.float64))


def test_special_values():
    assert A.affinity(np.float32(0.0)) == np.float32(np.sqrt(np.log(2.0)))
    # once e^-l < half an ulp of l, softplus(l) rounds to l
    for l in [np.float32(20.0), np.float32(50.5), np.float32(87.5), np.float32(1e6)]:
        assert A.softplus(l) == l
        assert A.affinity(l) == np.sqrt(l)
    # large negative logits: softplus ~ e^l; flushed to 0 below e^-87
    assert A.affinity(np.float32(-100.0)) == 0.0
    l = np.float32(-30.0)
    assert abs(float(A.softplus(l)) - np.exp(-30.0)) <= 2 * np.spacing(np.float32(np.exp(-30.0)))


def test_exp_neg_and_log1p_pieces():
    a = np.linspace(0, 87, 200001, dtype=np.float32)
    e = A.exp_neg(a)
    ref = np.exp(-a.astype(np.float64))
    assert _ulps(e, ref).max() <= 2.0
    u = np.linspace(0, 1, 200001, dtype=np.float32)
    g = A.log1p_small(u)
    ref = np.log1p(u.astype(np.float64))
    ok = u > 0
    assert _ulps(g[ok], ref[ok]).max() <= 4.0
    assert A.log1p_small(np.float32(0.0)) == 0.0


def test_sign_of_zero_logit_irrelevant():
    assert A.affinity(np.float32(-0.0)) == A.affinity(np.float32(0.0))
