"""The persistent expert products under concurrency and graph capture.

Their work-groups take tiles from device-side ticket counters; each launch
uses the next of 16 counter sets and leaves it cleared.  These tests run
launches on four streams at once and replay a captured layer forward, and
require every result to equal the same computation run alone, bit for bit
(each tile is computed by one work-group in a fixed K order, so the schedule
cannot change a value)."""
import numpy as np
import pytest
import torch

import moe_expert_routing_sqrt_amd as M
from moe_inputs import configs as C, generate as gen
from gpu_util import dev_i32, need_gpu

pytestmark = pytest.mark.gpu

COUNTS = [0, 1, 300, 257, 129, 700, 64, 511]


def _case(seed, d, d_ff, dtype, dev):
    g = torch.Generator(device=dev).manual_seed(seed)
    n, rows = len(COUNTS), sum(COUNTS)
    x = torch.randn((rows, d), generator=g, device=dev).to(torch.bfloat16)
    w13 = 0.05 * torch.randn((n, 2 * d_ff, d), generator=g, device=dev)
    w2 = 0.05 * torch.randn((n, d, d_ff), generator=g, device=dev)
    off = dev_i32(np.concatenate([[0], np.cumsum(COUNTS)]).astype(np.int32), dev)
    if dtype == M.MOE_E4M3:
        xq, xs = M.quantize_rows_e4m3(x)
        q13, s13 = M.quantize_blocks_e4m3(w13)
        q2, s2 = M.quantize_blocks_e4m3(w2)
        args = dict(xp=xq, w13=q13, w2=q2, dtype=dtype, xp_scale=xs, w13_scale=s13, w2_scale=s2)
    else:
        args = dict(xp=x, w13=w13.to(torch.bfloat16), w2=w2.to(torch.bfloat16), dtype=dtype)
    return off, rows, args


def _run(off, rows, args):
    yp, h, hs = M.expert_ffn(off, rows, args["xp"], args["w13"], args["w2"], args["dtype"],
                             xp_scale=args.get("xp_scale"), w13_scale=args.get("w13_scale"),
                             w2_scale=args.get("w2_scale"))
    return yp


@pytest.mark.parametrize("dtype", [M.MOE_BF16, M.MOE_E4M3])
def test_expert_ffn_on_four_streams(dtype):
    dev = need_gpu()
    print(f"expert ffn on 4 streams, dtype={dtype}", flush=True)
    d, d_ff = 1024, 512
    cases = [_case(11 + i, d, d_ff, dtype, dev) for i in range(4)]
    ref = [_run(*c).clone() for c in cases]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in cases]
    main = torch.cuda.current_stream()
    outs = [[] for _ in cases]
    for s in streams:
        s.wait_stream(main)
    for rep in range(3):
        for i, (c, s) in enumerate(zip(cases, streams)):
            with torch.cuda.stream(s):
                outs[i].append(_run(*c))
    torch.cuda.synchronize()
    for i, c in enumerate(cases):
        rows = c[1]
        for y in outs[i]:
            assert torch.equal(y[:rows], ref[i][:rows]), i


def test_layer_forward_graph_replay():
    """A captured forward replays into the layer's buffers after eager work on
    another input has overwritten them, each replay equal to the eager result."""
    dev = need_gpu()
    cfg = C.get("flash").with_(T=512, d=512, E=16, G=4, k=4, M=2, d_ff=256)
    print(f"graph replay T={cfg.T} d={cfg.d} E={cfg.E} d_ff={cfg.d_ff}", flush=True)
    inp = gen.make_router(cfg, device=dev)
    ex = gen.make_experts(cfg, device=dev)
    layer = M.MoELayer(cfg.T, cfg.d, cfg.E, cfg.G, cfg.M, cfg.k, cfg.d_ff, cfg.dtype, inp["w_gate"], inp["bias"],
                       ex["w13"], ex["w2"], ex["sh_w13"], ex["sh_w2"], group_topk=cfg.gk)
    x = inp["x"].clone()
    x2 = (inp["x"].float() * -0.5).to(inp["x"].dtype)
    eager = layer.forward(x).clone()
    eager2 = layer.forward(x2).clone()
    assert not torch.equal(eager, eager2)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out_g = layer.forward(x)
    for rep in range(3):
        layer.forward(x2)              # eager work that overwrites every internal buffer
        out_g.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, eager), rep
