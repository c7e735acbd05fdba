"""The persistent expert products under concurrency and graph capture.

Their work-groups take tiles from ticket counters in the caller's workspace
(zero-filled once; every call leaves it zero).  These tests run launches on
four streams at once, each stream with its own workspace, replay two captured
graphs concurrently on two streams, and replay a captured layer forward; every
result must equal the same computation run alone, bit for bit (each tile is
computed by one work-group in a fixed K order, so the schedule cannot change a
value)."""
import numpy as np
import pytest
import torch

import moe_expert_routing_sqrt_amd as M
from moe_inputs import configs as C, generate as gen
from gpu_util import cu_mask_stream, dev_i32, need_gpu

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


def _run(off, rows, args, ws=None, h=None, h_scale=None, yp=None):
    yp, h, hs = M.expert_ffn(off, rows, args["xp"], args["w13"], args["w2"], args["dtype"],
                             xp_scale=args.get("xp_scale"), w13_scale=args.get("w13_scale"),
                             w2_scale=args.get("w2_scale"), ws=ws, h=h, h_scale=h_scale, yp=yp)
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
    wss = [M.workspace(M.MOE_OP_EXPERT_FFN, None, dtype, dev) for _ in cases]
    outs = [[] for _ in cases]
    for s in streams:
        s.wait_stream(main)
    for rep in range(3):
        for i, (c, s) in enumerate(zip(cases, streams)):
            with torch.cuda.stream(s):
                outs[i].append(_run(*c, ws=wss[i]))
    torch.cuda.synchronize()
    for i, c in enumerate(cases):
        rows = c[1]
        for y in outs[i]:
            assert torch.equal(y[:rows], ref[i][:rows]), i


@pytest.mark.parametrize("dtype", [M.MOE_BF16, M.MOE_E4M3])
def test_expert_ffn_on_cu_masked_streams(dtype):
    """Persistent launches size their grid by the stream's CU mask: on a
    stream limited to 240 CUs and on one limited to 16 (two per XCD), each
    beside the other, the products equal the whole-chip ones bit for bit."""
    dev = need_gpu()
    n_cus = torch.cuda.get_device_properties(0).multi_processor_count
    print(f"expert ffn on CU-masked streams, dtype={dtype}, {n_cus} CUs", flush=True)
    words = (n_cus + 31) // 32
    res = [0] * words
    for x in range(min(8, words)):
        res[x] = 3 << (2 * x)  # bits x*32 + 2x, x*32 + 2x + 1
    rest = [(~r) & 0xFFFFFFFF for r in res]
    big, small = cu_mask_stream(torch, rest), cu_mask_stream(torch, res)
    d, d_ff = 1024, 512
    cases = [_case(21 + i, d, d_ff, dtype, dev) for i in range(2)]
    ref = [_run(*c).clone() for c in cases]
    torch.cuda.synchronize()
    main = torch.cuda.current_stream()
    wss = [M.workspace(M.MOE_OP_EXPERT_FFN, None, dtype, dev) for _ in cases]
    outs = [[], []]
    for s in (big, small):
        s.wait_stream(main)
    for rep in range(2):
        for i, s in enumerate((big, small)):
            with torch.cuda.stream(s):
                outs[i].append(_run(*cases[i], ws=wss[i]))
    torch.cuda.synchronize()
    for i, c in enumerate(cases):
        for y in outs[i]:
            assert torch.equal(y[:c[1]], ref[i][:c[1]]), i


@pytest.mark.parametrize("dtype", [M.MOE_BF16, M.MOE_E4M3])
def test_two_graphs_replayed_concurrently(dtype):
    """Two captures of the same expert products, each with its own workspace
    and buffers, replayed at the same time on two streams (three rounds, eager
    work between them): every replay equals the eager result."""
    dev = need_gpu()
    print(f"two graphs on two streams, dtype={dtype}", flush=True)
    d, d_ff = 1024, 512
    off, rows, args = _case(21, d, d_ff, dtype, dev)
    ref = _run(off, rows, args).clone()
    torch.cuda.synchronize()
    store = torch.uint8 if dtype == M.MOE_E4M3 else torch.bfloat16
    bufs = []
    for _ in range(2):
        ws = M.workspace(M.MOE_OP_EXPERT_FFN, None, dtype, dev)
        h = torch.empty((rows, d_ff), dtype=store, device=dev)
        hs = torch.empty((d_ff // 128, rows), dtype=torch.float32, device=dev) if dtype == M.MOE_E4M3 else None
        yp = torch.empty((rows, d), dtype=torch.bfloat16, device=dev)
        bufs.append((ws, h, hs, yp))
    torch.cuda.synchronize()
    graphs = []
    for ws, h, hs, yp in bufs:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            _run(off, rows, args, ws=ws, h=h, h_scale=hs, yp=yp)
        graphs.append(g)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in graphs]
    for rep in range(3):
        for _, _, _, yp in bufs:
            yp.zero_()
        _run(off, rows, args)                      # eager work between the replays
        main = torch.cuda.current_stream()
        for s in streams:
            s.wait_stream(main)
        for g, s in zip(graphs, streams):
            with torch.cuda.stream(s):
                g.replay()
        torch.cuda.synchronize()
        for i, (_, _, _, yp) in enumerate(bufs):
            assert torch.equal(yp[:rows], ref[:rows]), (rep, i)


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
