"""Every stage of the layer forward is deterministic by construction: no
floating-point atomics (the histogram counts are integer adds), each output
element of the products is computed by one work-group in a fixed K order, and
the selection, permutation and combine follow fixed orders.  These tests run
the whole forward 100 times and compare every intermediate and the output bit
for bit with the first run."""
import pytest
import torch

import moe_expert_routing_sqrt_amd as M
from moe_inputs import configs as C, generate as gen
from gpu_util import need_gpu

pytestmark = pytest.mark.gpu


def _snapshot(layer, out):
    b = layer.dbufs
    snap = {"logits": layer.logits, "idx": layer.idx, "w": layer.topk_w, "block_counts": layer.block_counts,
            "counts": b["counts"], "offsets": b["offsets"], "dest": b["dest"], "src": b["src"],
            "xp": b["xp"], "h": layer.h, "yp": layer.yp, "out": out}
    if b.get("xp_scale") is not None:
        snap["xp_scale"] = b["xp_scale"]
    if getattr(layer, "ysh", None) is not None:
        snap["ysh"] = layer.ysh
    return snap


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", ["flash", "v3", "v3_fp8", "v3_skew_ep0"])
def test_layer_forward_100_repeats_bitwise(name):
    dev = need_gpu()
    cfg = C.get(name)
    print(f"determinism {name}: 100 forwards", flush=True)
    inp = gen.make_router(cfg, device=dev)
    ex = gen.make_experts(cfg, device=dev)
    layer = M.MoELayer(cfg.T, cfg.d, cfg.E, cfg.G, cfg.M, cfg.k, cfg.d_ff, cfg.dtype, inp["w_gate"],
                       inp["bias"], ex["w13"], ex["w2"], ex["sh_w13"], ex["sh_w2"],
                       logit_offset=inp["logit_offset"], e_begin=cfg.e_begin, e_end=cfg.e_end,
                       group_topk=cfg.gk)
    del ex
    out = layer.forward(inp["x"])
    first = {k: v.clone() for k, v in _snapshot(layer, out).items()}
    rows = int(first["offsets"][-1].item())
    for rep in range(99):
        out = layer.forward(inp["x"])
        for k, v in _snapshot(layer, out).items():
            a, b = first[k], v
            if k in ("xp", "h", "yp"):
                a, b = a[:rows], b[:rows]      # rows past the packed ones are never written
            if k == "xp_scale":
                a, b = a[:, :rows], b[:, :rows]
            assert torch.equal(a, b), (rep + 1, k)
        if rep % 33 == 32:
            print(f"  {rep + 2} forwards equal", flush=True)
    torch.cuda.synchronize()
