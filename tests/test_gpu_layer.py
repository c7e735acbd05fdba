"""GPU parity, end to end (S6): the whole layer through MoELayer (the launch
configuration the benchmark times) against the oracle, each side forming its
own logits.  A near-tie in the logits may flip a token's selection; such
tokens are counted and their score gaps checked, and the output error is
measured on the tokens whose routing matches."""
import numpy as np
import pytest
import torch

import moe_expert_routing_sqrt_amd as M
from moe_inputs import configs as C, generate as gen
from oracle import combine as OC, dispatch as OD, ffn as OF, route as OR

from gpu_util import expert_host, host, need_gpu, rel_max_err, router_inputs

pytestmark = pytest.mark.gpu


def _layer(cfg, inp, ex):
    return M.MoELayer(cfg.T, cfg.d, cfg.E, cfg.G, cfg.M, cfg.k, cfg.d_ff, cfg.dtype, inp["w_gate"],
                      inp["bias"], ex["w13"], ex["w2"], ex["sh_w13"], ex["sh_w2"],
                      logit_offset=inp["logit_offset"], e_begin=cfg.e_begin, e_end=cfg.e_end,
                      group_topk=cfg.gk)


def _flips(idx_gpu, o, cfg):
    bad = np.nonzero((idx_gpu != o["idx"]).any(1))[0]
    return bad


@pytest.mark.parametrize("name", ["tiny", "flash"])
def test_layer_end_to_end(name):
    dev = need_gpu()
    cfg, inp, o = router_inputs(name)
    print(f"layer S6 {name}", flush=True)
    ex = gen.make_experts(cfg, device=dev)
    layer = _layer(cfg, inp, ex)
    out = host(layer.forward(inp["x"]))
    torch.cuda.synchronize()
    idx_g = host(layer.idx)
    bad = _flips(idx_g, o, cfg)
    print(f"  routing flips vs oracle logits: {len(bad)} of {cfg.T}")
    assert len(bad) <= max(1, cfg.T // 1000)
    counts, offsets, dest, src = OD.dispatch(o["idx"], cfg.E)
    yp, _ = OF.grouped_ffn(OD.pack(o["x"], src), offsets, host(ex["w13"]), host(ex["w2"]))
    ysh, _ = OF.expert_forward(o["x"], host(ex["sh_w13"][0]), host(ex["sh_w2"][0]))
    ref = OC.combine(yp, dest, o["w"], ysh=ysh)
    ok = np.ones(cfg.T, bool)
    ok[bad] = False
    err = rel_max_err(out[ok], ref[ok])
    print(f"  rel max err {err:.3e}")
    assert err <= (1e-5 if cfg.dtype == "f32" else 2e-2)


def test_layer_v3_sampled_tokens():
    dev = need_gpu()
    cfg, inp, o = router_inputs("v3")
    print("layer S6 v3 (sampled tokens)", flush=True)
    ex = gen.make_experts(cfg, device=dev)
    layer = _layer(cfg, inp, ex)
    out_d = layer.forward(inp["x"])
    torch.cuda.synchronize()
    idx_g = host(layer.idx)
    bad = _flips(idx_g, o, cfg)
    print(f"  routing flips vs oracle logits: {len(bad)} of {cfg.T}")
    assert len(bad) <= cfg.T // 1000
    rng = np.random.default_rng(0)
    toks = [int(t) for t in rng.choice(cfg.T, 6, replace=False) if t not in set(bad.tolist())]
    toks += [cfg.T - 1]
    out = host(out_d[torch.tensor(toks, device=dev)])
    sh13, sh2 = expert_host(cfg, 0, dev, shared=True)
    refs = []
    for t in toks:
        x = o["x"][t:t + 1]
        y, _ = OF.expert_forward(x, sh13, sh2)
        for j in range(cfg.k):
            e = int(o["idx"][t, j])
            w13, w2 = host(ex["w13"][e]), host(ex["w2"][e])
            ye, _ = OF.expert_forward(x, w13, w2)
            y = y + float(o["w"][t, j]) * ye
        refs.append(y[0])
    err = rel_max_err(out, np.stack(refs))
    print(f"  sampled tokens {toks} rel max err {err:.3e}")
    assert err <= 2e-2
    del layer, ex
    torch.cuda.empty_cache()


def test_layer_skew_local_share():
    """One expert-parallel rank's 4 experts under Zipf routing skew, fp32
    scatter-add output."""
    dev = need_gpu()
    cfg, inp, o = router_inputs("v3_skew_ep0")
    print("layer S6 v3_skew_ep0", flush=True)
    ex = gen.make_experts(cfg, device=dev)          # the local experts only
    layer = _layer(cfg, inp, ex)
    layer.out.zero_()
    out = host(layer.forward(inp["x"]))
    torch.cuda.synchronize()
    assert layer.out.dtype == torch.float32
    counts, offsets, dest, src = OD.dispatch(o["idx"], cfg.E, cfg.e_begin, cfg.e_end)
    print(f"  local rows per expert {counts.tolist()}")
    idx_g = host(layer.idx)
    bad = _flips(idx_g, o, cfg)
    assert len(bad) <= cfg.T // 1000
    yp, _ = OF.grouped_ffn(OD.pack(o["x"], src), offsets, host(ex["w13"]), host(ex["w2"]))
    ref = OC.combine(yp, dest, o["w"], out_init=np.zeros((cfg.T, cfg.d)))
    ok = np.ones(cfg.T, bool)
    ok[bad] = False
    err = rel_max_err(out[ok], ref[ok])
    print(f"  rel max err {err:.3e}")
    assert err <= 2e-2
