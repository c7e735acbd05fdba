"""Pins for the oracle's router (gate logits, node-limited top-k, weights)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import route as R
from moe_inputs import configs as C, generate as gen
import brute

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _f32(v):
    return np.asarray(v, dtype=np.float32)


def test_worked_examples():
    g = json.load(open(os.path.join(GOLD, "route_worked.json")))
    for case in g["cases"]:
        s = _f32([case["s"]])
        b = s + _f32([case["bias"]])
        idx, w, gmask = R.select(s, b, g["G"], g["M"], g["k"], g["gk"])
        assert idx[0].tolist() == case["idx"], case["name"]
        exp_w = [np.float32(float(Fraction(f))) for f in case["w"]]
        # fp32(s_j / S) of exact dyadic values is the correctly rounded fraction
        assert w[0].tolist() == [float(v) for v in exp_w], case["name"]
        assert sorted(np.nonzero(gmask[0])[0].tolist()) == case["groups"]


def _dyadic(rng, shape, lo=-0.5, hi=1.5, bits=6):
    """Values on a coarse dyadic grid: many exact ties, and every fp32 sum of
    a few of them is exact."""
    q = 2.0 ** -bits
    n = int((hi - lo) / q)
    return (lo + q * rng.integers(0, n, size=shape)).astype(np.float32)


@pytest.mark.parametrize("E,G,M,k", [(16, 4, 2, 4), (8, 4, 2, 3), (12, 3, 2, 5), (16, 4, 4, 6),
                                     (8, 2, 1, 2), (16, 8, 3, 5), (9, 3, 3, 1), (16, 1, 1, 3)])
def test_brute_force_dyadic(E, G, M, k):
    rng = np.random.default_rng(1000 + E * 31 + G * 7 + M * 3 + k)
    gk = -(-k // M)
    if gk > E // G:
        pytest.skip("gk exceeds group size")
    T = 60
    s = np.abs(_dyadic(rng, (T, E)))
    bias = _dyadic(rng, (T, E), -0.25, 0.25, 4)
    b = (s + bias).astype(np.float32)
    idx, w, gmask = R.select(s, b, G, M, k, gk)
    for t in range(T):
        ordered, bw, groups = brute.select_token(s[t], b[t], G, M, k, gk)
        assert idx[t].tolist() == list(ordered), (t, b[t])
        assert sorted(np.nonzero(gmask[t])[0].tolist()) == list(groups)
        for j in range(k):
            assert abs(Fraction(float(w[t, j])) - bw[j]) <= Fraction(float(np.spacing(np.float32(bw[j])))) * k


def test_brute_force_tiny_config_scores():
    """The tiny workload's own inputs: oracle selection == enumeration."""
    cfg = C.TINY
    inp = gen.make_router(cfg)
    L = R.gate_logits(inp["x"].numpy(), inp["w_gate"].numpy())
    s, b = R.scores(L, inp["bias"].numpy())
    idx, w, _ = R.select(s, b, cfg.G, cfg.M, cfg.k, cfg.gk)
    for t in range(cfg.T):
        ordered, bw, _ = brute.select_token(s[t], b[t], cfg.G, cfg.M, cfg.k, cfg.gk)
        assert idx[t].tolist() == list(ordered)


def _invariants(idx, w, E, G, M, k):
    T = idx.shape[0]
    assert idx.shape == (T, k)
    assert np.all((idx >= 0) & (idx < E))
    srt = np.sort(idx, axis=1)
    assert np.all(srt[:, 1:] != srt[:, :-1]), "experts per token must be distinct"
    groups = idx // (E // G)
    ng = np.array([len(set(r)) for r in groups.tolist()])
    assert ng.max() <= M, "a token reached more than M groups"
    assert np.all(w >= 0)
    ssum = w.astype(np.float64).sum(1)
    assert np.all(np.abs(ssum - 1.0) <= k * 2 ** -23 * 2)


@pytest.mark.parametrize("name,T", [("tiny", 256), ("flash", 512), ("v3", 256), ("v3_skew_ep0", 256)])
def test_invariants_on_workloads(name, T):
    cfg = C.get(name).with_(T=T)
    inp = gen.make_router(cfg)
    off = None if inp["logit_offset"] is None else inp["logit_offset"].numpy()
    L, idx, w = R.route(inp["x"].float().numpy(), inp["w_gate"].numpy(), inp["bias"].numpy(),
                        cfg.G, cfg.M, cfg.k, cfg.gk, off)
    _invariants(idx, w, cfg.E, cfg.G, cfg.M, cfg.k)
    # weights are proportional to the unbiased affinities of the chosen experts
    s, _ = R.scores(L, inp["bias"].numpy(), off)
    sel = np.take_along_axis(s, idx, 1).astype(np.float64)
    ratio = w / sel
    assert np.allclose(ratio, ratio[:, :1], rtol=4e-7)


def test_textbook_special_cases():
    rng = np.random.default_rng(7)
    T, E, k = 200, 16, 4
    L = rng.standard_normal((T, E)).astype(np.float32)
    zero = np.zeros(E, np.float32)
    # one group (or all groups kept), no bias: top-k of the logits themselves,
    # since sqrt(softplus(.)) is increasing
    ref = np.argsort(-L, axis=1, kind="stable")[:, :k]
    for G, M in [(1, 1), (4, 4), (16, 16)]:
        idx, w = R.route_from_logits(L, zero, G, M, k, -(-k // M))
        assert np.array_equal(idx, ref), (G, M)
    # k = 1: argmax
    idx, w = R.route_from_logits(L, zero, 1, 1, 1, 1)
    assert np.array_equal(idx[:, 0], np.argmax(L, axis=1))
    assert np.all(w == 1.0)


def test_gate_logits_forward_error_bound():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 512)).astype(np.float32)
    W = (0.02 * rng.standard_normal((512, 32))).astype(np.float32)
    L = R.gate_logits(x, W)
    exact = np.array([[float(sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x[i], W[:, j])))
                       for j in range(0, 32, 7)] for i in range(0, 64, 9)])
    got = L[::9, ::7].astype(np.float64)
    # one fp32 rounding of the exact value (fp64 accumulation error is far below)
    assert np.all(np.abs(got - exact) <= np.spacing(np.abs(got).astype(np.float32)) * 0.5 + 1e-12)


def test_logit_offset_is_added_before_affinity():
    cfg = C.V3_SKEW_EP0
    off = gen.zipf_logit_offset(cfg.E).numpy()
    assert off[0] == pytest.approx(2.0) and off[-1] == pytest.approx(0.0, abs=1e-7)
    assert np.all(np.diff(off) <= 0)
    L = np.zeros((1, cfg.E), np.float32)
    s, b = R.scores(L, np.zeros(cfg.E, np.float32), off)
    s2, _ = R.scores(off[None, :], np.zeros(cfg.E, np.float32))
    assert np.array_equal(s, s2)
