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


@pytest.mark.parametrize("name,T", [("tiny", None), ("flash", None), ("v3", None), ("v3", 1000), ("flash", 77)])
def test_gate_logits_tolerance(name, T):
    """Full sizes, and token counts that end in a partial 128- or 64-row tile."""
    dev = need_gpu()
    cfg, inp, o = router_inputs(name, T)
    print(f"route S1 {name} T={cfg.T}", flush=True)
    sh = moe_shape(cfg)
    w_prep = M.gate_prepare(inp["w_gate"])
    L, idx, w, bc = M.route(sh, inp["x"], w_prep, inp["bias"], inp["logit_offset"])
    torch.cuda.synchronize()
    err = logits_row_err(host(L), o["L"])
    print(f"  worst-row logit error {err:.3e}")
    assert err <= 1e-5
    # routing from the GPU's own logits is the oracle's routing of those logits
    gi, gw = OR.route_from_logits(host(L), o["bias"], cfg.G, cfg.M, cfg.k, cfg.gk, o["offset"])
    assert np.array_equal(host(idx), gi)
    assert np.array_equal(host(w).view(np.uint32), gw.view(np.uint32))


def test_gate_prepare_planes_exact():
    dev = need_gpu()
    cfg, inp, o = router_inputs("v3")
    w_prep = M.gate_prepare(inp["w_gate"])
    torch.cuda.synchronize()
    p = host(w_prep).astype(np.float32)           # [3, E, d] bf16 values
    s = (p[0] + p[1]) + p[2]
    assert np.array_equal(s, o["w_gate"].T)


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
    w_prep = M.gate_prepare(inp["w_gate"])
    outs = []
    for _ in range(3):
        L, idx, w, bc = M.route(sh, inp["x"], w_prep, inp["bias"])
        outs.append((L.clone(), idx.clone(), w.clone(), bc.clone()))
    torch.cuda.synchronize()
    for rep in outs[1:]:
        for a, b in zip(outs[0], rep):
            assert torch.equal(a, b)
