"""GPU parity: gate logits (S1) and routing from the same fp32 logits (S2).

Routing must match the oracle bit for bit given the same logits; gate logits
must match within 1e-5 relative (per row, normwise) of the oracle's fp64-formed
logits."""
import numpy as np
import pytest
import torch

import moe_expert_routing_sqrt_amd as M
from moe_inputs import configs as C
from oracle import route as OR

from gpu_util import (block_counts, dev_f32, host, logits_row_err, moe_shape, need_gpu,
                      router_inputs)

pytestmark = pytest.mark.gpu


def _route_in(cfg, L, bias, offset, dev):
    sh = moe_shape(cfg)
    logits = dev_f32(L, dev)
    off = None if offset is None else dev_f32(offset, dev)
    _, idx, w, bc = M.route(sh, None, None, dev_f32(bias, dev), off, logits=logits, logits_in=True)
    torch.cuda.synchronize()
    return host(idx), host(w), host(bc)


@pytest.mark.parametrize("name,T", [("tiny", None), ("flash", None), ("v3", None), ("v3_skew_ep0", None),
                                    ("v3", 1000), ("flash", 1), ("tiny", 63)])
def test_route_bitexact_from_oracle_logits(name, T):
    dev = need_gpu()
    cfg, inp, o = router_inputs(name, T)
    print(f"route S2 {name} T={cfg.T}", flush=True)
    idx, w, bc = _route_in(cfg, o["L"], o["bias"], o["offset"], dev)
    assert np.array_equal(idx, o["idx"])
    assert np.array_equal(w.view(np.uint32), o["w"].view(np.uint32))
    assert np.array_equal(bc, block_counts(o["idx"], cfg.E))


@pytest.mark.timeout(400)
@pytest.mark.parametrize("name,T", [("tiny", None), ("flash", None), ("v3", None), ("v3", 1000), ("flash", 77),
                                    ("v3", 1), ("v3", 300), ("v3_skew_ep0", 4100),
                                    ("v3", 20000), ("v3", 32768), ("v3", 65536)])
def test_gate_logits_tolerance(name, T):
    """Full sizes, and token counts that end in a partial 256-, 128- or 64-row
    tile.  At E = 256 with bf16 x the gate product is split over its reduction
    into partial products that the selection sums: 4 at V3 (64 row tiles), 8
    at 1, 300, 1000 and 4100 tokens, 3 at 20000, 2 at 32768, and none at 65536
    tokens (256 row tiles fill the chip; the product writes the logits).  At
    E = 64 (Flash) the 64 x 64-tile product splits the same way: 4 partial
    products at 4096 tokens, 8 at 77."""
    dev = need_gpu()
    cfg, inp, o = router_inputs(name, T)
    print(f"route S1 {name} T={cfg.T}", flush=True)
    sh = moe_shape(cfg)
    L, idx, w, bc = M.route(sh, inp["x"], inp["w_gate"], inp["bias"], inp["logit_offset"])
    torch.cuda.synchronize()
    err = logits_row_err(host(L), o["L"])
    print(f"  worst-row logit error {err:.3e}")
    assert err <= 1e-5
    # routing from the GPU's own logits is the oracle's routing of those logits
    gi, gw = OR.route_from_logits(host(L), o["bias"], cfg.G, cfg.M, cfg.k, cfg.gk, o["offset"])
    assert np.array_equal(host(idx), gi)
    assert np.array_equal(host(w).view(np.uint32), gw.view(np.uint32))


@pytest.mark.parametrize("name,T", [("flash", None), ("v3", 1000)])
def test_logits_kept_in_workspace(name, T):
    """logits = NULL: the route keeps them (or, split, their partial
    products) in its workspace; the selection is the same as with a logits
    buffer."""
    dev = need_gpu()
    cfg, inp, o = router_inputs(name, T)
    sh = moe_shape(cfg)
    ws = M.workspace(M.MOE_OP_ROUTE, sh, M.MOE_BF16, dev)
    L, idx, w, bc = M.route(sh, inp["x"], inp["w_gate"], inp["bias"], ws=ws)
    L2, idx2, w2, bc2 = M.route(sh, inp["x"], inp["w_gate"], inp["bias"], ws=ws, keep_logits=False)
    torch.cuda.synchronize()
    assert L2 is None
    assert torch.equal(idx, idx2) and torch.equal(w, w2) and torch.equal(bc, bc2)


def _special_logits(rng, T, E):
    sp = np.array([0.0, -0.0, 1e-30, -1e-30, 1e-40, -1e-40, 1.4e-45, -1.4e-45, 86.9, -86.9, 87.0, -87.0,
                   87.5, -87.5, 88.0, -88.0, 100.0, -100.0, 1e30, -1e30, 3.4e38, -3.4e38, 0.5, -0.5,
                   np.log(2.0), 20.0, -20.0, 1e-7, -1e-7, 15.9424, -15.9424, 0.34657], dtype=np.float32)
    L = rng.uniform(-30, 30, size=(T, E)).astype(np.float32)
    flat = L.reshape(-1)
    flat[: sp.size * 8] = np.tile(sp, 8)
    rng.shuffle(flat[: sp.size * 8 * 2])
    return L


def test_affinity_bitexact_all_experts_selected():
    """k = E, M = G: the weights are s_j / sum(s) over every expert, so a
    single differing affinity bit shows up."""
    dev = need_gpu()
    cfg = C.TINY.with_(T=512, k=16, M=4)
    rng = np.random.default_rng(11)
    L = _special_logits(rng, cfg.T, cfg.E)
    bias = np.zeros(cfg.E, np.float32)
    idx_o, w_o = OR.route_from_logits(L, bias, cfg.G, cfg.M, cfg.k, cfg.gk)
    idx, w, _ = _route_in(cfg, L, bias, None, dev)
    assert np.array_equal(idx, idx_o)
    assert np.array_equal(w.view(np.uint32), w_o.view(np.uint32))


def _dense_affinity_logits():
    """About 1M fp32 logits: a strided sweep over every fp32 in [-200, 88],
    runs of consecutive values at the places where the affinity's evaluation
    changes form or rounds close to a boundary (0, +-2^-14, the fp32 midpoint
    crossing near -8.5e-9, +-1, +-20, +-87, +-150), and special values (rows
    are 16 neighbours of the list, so no row has only zero affinities, for
    which the weights would be 0/0)."""
    lo, hi = np.float32(-200.0).view(np.uint32), np.float32(88.0).view(np.uint32)
    neg = np.arange(0x80000000, int(lo) + 1, 4099, dtype=np.uint64).astype(np.uint32).view(np.float32)
    pos = np.arange(0, int(hi) + 1, 4099, dtype=np.uint64).astype(np.uint32).view(np.float32)
    runs = []
    for c in (0.0, 2.0 ** -14, -(2.0 ** -14), -8.5e-9, 1.0, -1.0, 20.0, -20.0, 87.0, -87.0, 150.0, -150.0):
        b = np.int64(np.float32(c).view(np.uint32))
        runs.append((b + np.arange(-8192, 8192)).astype(np.uint32).view(np.float32))
    sp = np.array([0.0, -0.0, 1e-30, -1e-30, 1.4e-45, -1.4e-45, 300.0, -300.0, 301.0, -301.0, 3.4e38,
                   -3.4e38, 1e30, -1e30], dtype=np.float32)
    l = np.concatenate([neg, pos] + runs + [sp])
    l = l[np.isfinite(l)]
    return l


def test_affinity_bitexact_dense():
    """Every expert selected (k = E, M = G, zero bias): the order of each
    token's experts and the bits of w = s_j / sum(s) follow every affinity
    bit, over about a million logits chosen across the whole fp32 range."""
    dev = need_gpu()
    l = _dense_affinity_logits()
    E = 16
    T = -(-l.size // E)
    L = np.resize(l, T * E).reshape(T, E).astype(np.float32)
    cfg = C.TINY.with_(T=T, k=E, M=4)
    bias = np.zeros(E, np.float32)
    idx_o, w_o = OR.route_from_logits(L, bias, cfg.G, cfg.M, cfg.k, cfg.gk)
    idx, w, _ = _route_in(cfg, L, bias, None, dev)
    assert np.array_equal(idx, idx_o)
    assert np.array_equal(w.view(np.uint32), w_o.view(np.uint32))


def test_affinity_monotone_on_gpu():
    """Each token's 16 logits are consecutive fp32 values in ascending order;
    with every expert selected, the GPU's weight w_e = s_e / S must not
    decrease with e (the exact affinity is increasing)."""
    dev = need_gpu()
    E = 16
    starts = np.concatenate([np.linspace(-200, 80, 20000, dtype=np.float32),
                             np.float32(np.linspace(-1e-7, 1e-7, 4000)),
                             np.float32([2.0 ** -14, -(2.0 ** -14), -8.5e-9])])
    base = starts.view(np.uint32).astype(np.int64)
    neg = starts < 0
    step = np.where(neg, -1, 1)[:, None] * np.arange(E)[None, :]
    L = (base[:, None] + step).astype(np.uint32).view(np.float32)
    L = np.sort(L, axis=1)
    T = L.shape[0]
    cfg = C.TINY.with_(T=T, k=E, M=4)
    idx, w, _ = _route_in(cfg, L, np.zeros(E, np.float32), None, dev)
    we = np.zeros((T, E), np.float32)
    np.put_along_axis(we, idx.astype(np.int64), w, axis=1)
    assert np.all(np.diff(we.astype(np.float64), axis=1) >= 0)


@pytest.mark.parametrize("E,G,M,k", [(16, 4, 2, 4), (64, 8, 4, 6), (256, 8, 4, 8), (256, 8, 1, 3),
                                     (64, 1, 1, 4), (128, 4, 3, 7), (32, 8, 8, 16),
                                     (256, 64, 8, 8), (128, 32, 4, 8), (64, 2, 2, 8), (256, 2, 2, 8)])
def test_adversarial_ties(E, G, M, k):
    """Dyadic logits with many exact ties and negative biased scores.  The
    shapes give a group every lane width the kernel reduces over: 1, 2, 4, 8,
    16, 32 and 64 lanes (experts per group / experts per lane)."""
    dev = need_gpu()
    rng = np.random.default_rng(E + 7 * M + k)
    T = 300
    cfg = C.TINY.with_(T=T, E=E, G=G, M=M, k=k)
    L = (rng.integers(-8, 9, size=(T, E)) * 0.25).astype(np.float32)
    L[:5] = 0.0                                            # all equal
    bias = (rng.integers(-4, 5, size=E) * 0.25).astype(np.float32)
    bias[: E // 2] -= 2.0                                  # negative biased scores
    idx_o, w_o = OR.route_from_logits(L, bias, G, M, k, cfg.gk)
    idx, w, bc = _route_in(cfg, L, bias, None, dev)
    assert np.array_equal(idx, idx_o)
    assert np.array_equal(w.view(np.uint32), w_o.view(np.uint32))
    assert np.array_equal(bc, block_counts(idx_o, E))


def test_route_deterministic_repeat():
    dev = need_gpu()
    cfg, inp, o = router_inputs("v3")
    sh = moe_shape(cfg)
    outs = []
    for _ in range(3):
        L, idx, w, bc = M.route(sh, inp["x"], inp["w_gate"], inp["bias"])
        outs.append((L.clone(), idx.clone(), w.clone(), bc.clone()))
    torch.cuda.synchronize()
    for rep in outs[1:]:
        for a, b in zip(outs[0], rep):
            assert torch.equal(a, b)
