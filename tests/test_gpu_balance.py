"""GPU parity: per-expert bias update (moe_bias_update) against the oracle.

The update is integer counting plus one fp32 add per expert, so the bias and
the load must match the oracle bit for bit, also along an iterated
route -> update loop (each step is exact, so the trajectories stay identical)."""
import numpy as np
import pytest
import torch

import moe_expert_routing_sqrt_amd as M
from oracle import balance as OB
from oracle import route as OR

from gpu_util import dev_f32, dev_i32, host, moe_shape, need_gpu, router_inputs

pytestmark = pytest.mark.gpu


def _bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


@pytest.mark.parametrize("name", ["tiny", "flash", "v3", "v3_skew_ep0"])
@pytest.mark.parametrize("gamma", [1e-3, 0.25])
def test_update_from_route_block_counts(name, gamma):
    dev = need_gpu()
    cfg, inp, o = router_inputs(name)
    print(f"bias update {name} gamma={gamma}", flush=True)
    sh = moe_shape(cfg)
    bias = dev_f32(o["bias"], dev)
    off = None if o["offset"] is None else dev_f32(o["offset"], dev)
    _, idx, _, bc = M.route(sh, None, None, bias, off, logits=dev_f32(o["L"], dev), logits_in=True)
    load = M.bias_update(bc, bias, gamma)
    torch.cuda.synchronize()
    ref_load = OB.expert_load(o["idx"], cfg.E)
    assert np.array_equal(host(load), ref_load)
    assert np.array_equal(_bits(host(bias)), _bits(OB.bias_update(ref_load, o["bias"], gamma)))


def test_iterated_loop_matches_oracle_trajectory():
    dev = need_gpu()
    E, G, Mg, k, T = 64, 8, 4, 6, 1000            # ragged last route block
    gk = -(-k // Mg)
    sh = M.shape(T, 64, E, G, Mg, k, 32, gk)
    rng = np.random.default_rng(11)
    offset = (2.0 * (np.arange(E)[::-1] / (E - 1)) ** 3).astype(np.float32)
    bias_h = np.zeros(E, dtype=np.float32)
    bias_d = dev_f32(bias_h, dev)
    off_d = dev_f32(offset, dev)
    ratios = []
    for step in range(25):
        L = rng.normal(size=(T, E)).astype(np.float32)
        _, idx, _, bc = M.route(sh, None, None, bias_d, off_d, logits=dev_f32(L, dev), logits_in=True)
        load = M.bias_update(bc, bias_d, 0.02)
        torch.cuda.synchronize()
        ridx, _ = OR.route_from_logits(L, bias_h, G, Mg, k, gk, offset)
        rload = OB.expert_load(ridx, E)
        bias_h = OB.bias_update(rload, bias_h, 0.02)
        assert np.array_equal(host(idx), ridx), step
        assert np.array_equal(host(load), rload), step
        assert np.array_equal(_bits(host(bias_d)), _bits(bias_h)), step
        ratios.append(rload.max() / rload.mean())
    print(f"  max/mean load {ratios[0]:.2f} -> {ratios[-1]:.2f}")
    assert ratios[-1] < ratios[0]


@pytest.mark.parametrize("R,E", [(1, 1), (1, 256), (3, 64), (5000, 64), (257, 1024), (2, 7)])
def test_count_matrix_shapes(R, E):
    dev = need_gpu()
    rng = np.random.default_rng(R * 31 + E)
    counts = rng.integers(0, 9, size=(R, E)).astype(np.int32)
    if R == 2:
        counts[:] = 0                               # empty batch: nothing moves
    bias_h = rng.uniform(-1, 1, size=E).astype(np.float32)
    bias_d = dev_f32(bias_h, dev)
    load = M.bias_update(dev_i32(counts, dev), bias_d, 0.125)
    torch.cuda.synchronize()
    rload = counts.astype(np.int64).sum(0)
    assert np.array_equal(host(load), rload)
    assert np.array_equal(_bits(host(bias_d)), _bits(OB.bias_update(rload, bias_h, 0.125)))


def test_layer_update_bias_after_forward():
    dev = need_gpu()
    from moe_inputs import generate as gen
    cfg, inp, o = router_inputs("tiny")
    ex = gen.make_experts(cfg, device=dev)
    layer = M.MoELayer(cfg.T, cfg.d, cfg.E, cfg.G, cfg.M, cfg.k, cfg.d_ff, cfg.dtype, inp["w_gate"],
                       inp["bias"].clone(), ex["w13"], ex["w2"], ex["sh_w13"], ex["sh_w2"],
                       group_topk=cfg.gk)
    layer.forward(inp["x"])
    load = layer.update_bias(0.01)
    torch.cuda.synchronize()
    rload = OB.expert_load(o["idx"], cfg.E)         # the oracle's routing of the same batch
    assert np.array_equal(host(load), rload)
    assert np.array_equal(_bits(host(layer.bias)), _bits(OB.bias_update(rload, o["bias"], 0.01)))
