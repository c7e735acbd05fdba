"""GPU parity: grouped SwiGLU expert FFN from the oracle's packed rows (S4).
Outputs must be within 2e-2 relative max error (bf16) of the oracle's fp64
result; the fp32 path within 1e-5."""
import numpy as np
import pytest
import torch

import moe_expert_routing_sqrt_amd as M
from moe_inputs import configs as C, generate as gen
from oracle import dispatch as OD, ffn as OF

from gpu_util import dev_i32, host, need_gpu, rel_max_err, router_inputs

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-5}


def _ragged_case(dtype, d, d_ff, counts, seed):
    dev = need_gpu()
    g = torch.Generator(device=dev).manual_seed(seed)
    n_exp = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = int(offsets[-1])
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    xp = torch.randn((max(rows, 1), d), generator=g, device=dev).to(tdt)
    w13 = (0.05 * torch.randn((n_exp, 2 * d_ff, d), generator=g, device=dev)).to(tdt)
    w2 = (0.05 * torch.randn((n_exp, d, d_ff), generator=g, device=dev)).to(tdt)
    yp, h, _ = M.expert_ffn(dev_i32(offsets, dev), max(rows, 1), xp, w13, w2)
    torch.cuda.synchronize()
    ref, flops = OF.grouped_ffn(host(xp), offsets, host(w13), host(w2))
    assert flops == rows * 6 * d * d_ff
    return host(yp)[:rows], ref


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("counts", [
    [0, 1, 127, 128, 129, 300, 0, 5],      # ragged tails, empty experts
    [1],                                   # a single row
    [513, 0, 0, 255],
    [64] * 16 + [0, 1000],                 # many small experts and one hot one
    [33, 65, 97, 161, 193, 225, 256, 31],  # a tail in every 32-row band of a tile
])
def test_ragged_groups(dtype, counts):
    print(f"ffn ragged {dtype} {counts}", flush=True)
    got, ref = _ragged_case(dtype, 512, 256, counts, seed=len(counts) * 13 + sum(counts))
    err = rel_max_err(got, ref)
    print(f"  rel max err {err:.3e}")
    assert err <= TOL[dtype]


def test_ffn_odd_width_uses_vector_path():
    # d % 256 != 0: the matrix-core tiles do not apply; results stay correct
    got, ref = _ragged_case("bf16", 320, 96, [3, 70, 0, 129], seed=5)
    assert rel_max_err(got, ref) <= 2e-2


def test_ffn_narrow_hidden_width():
    # d_ff = 128: the down-projection's K is too short for the matrix-core
    # pipeline (it needs K >= 256); d_ff = 384: the smallest K of an odd
    # number of 128-column blocks that still takes it
    for d_ff, counts in ((128, [5, 300, 0, 17]), (384, [260, 1, 0, 511])):
        got, ref = _ragged_case("bf16", 256, d_ff, counts, seed=d_ff)
        assert rel_max_err(got, ref) <= 2e-2, d_ff


@pytest.mark.parametrize("name", ["tiny", "flash"])
def test_ffn_workload_full(name):
    """Every routed expert of the workload, from the oracle's packed rows."""
    dev = need_gpu()
    cfg, inp, o = router_inputs(name)
    print(f"ffn S4 {name}", flush=True)
    counts, offsets, dest, src = OD.dispatch(o["idx"], cfg.E)
    ex = gen.make_experts(cfg, device=dev)
    xp_h = OD.pack(o["x"], src)
    xp = inp["x"][torch.from_numpy(src.astype(np.int64)).to(dev)].contiguous()
    yp, _, _ = M.expert_ffn(dev_i32(offsets, dev), cfg.pairs, xp, ex["w13"], ex["w2"])
    torch.cuda.synchronize()
    ref, _ = OF.grouped_ffn(xp_h, offsets, host(ex["w13"]), host(ex["w2"]))
    err = rel_max_err(host(yp), ref)
    print(f"  rel max err {err:.3e}")
    assert err <= TOL[cfg.dtype]
    # shared expert: one group over all tokens, unpermuted
    ysh, _, _ = M.expert_ffn(dev_i32([0, cfg.T], dev), cfg.T, inp["x"], ex["sh_w13"], ex["sh_w2"])
    torch.cuda.synchronize()
    ref_sh, _ = OF.expert_forward(o["x"], host(ex["sh_w13"][0]), host(ex["sh_w2"][0]))
    assert rel_max_err(host(ysh), ref_sh) <= TOL[cfg.dtype]


def test_ffn_v3_sampled_experts():
    """V3 shapes at full size: all 256 experts run on the GPU; the oracle
    recomputes every row of a sample of experts (the busiest, the idlest and
    a spread in between)."""
    dev = need_gpu()
    cfg, inp, o = router_inputs("v3")
    print("ffn S4 v3 (sampled experts)", flush=True)
    counts, offsets, dest, src = OD.dispatch(o["idx"], cfg.E)
    ex = gen.make_experts(cfg, device=dev)
    xp = inp["x"][torch.from_numpy(src.astype(np.int64)).to(dev)].contiguous()
    yp, _, _ = M.expert_ffn(dev_i32(offsets, dev), cfg.pairs, xp, ex["w13"], ex["w2"])
    torch.cuda.synchronize()
    order = np.argsort(counts, kind="stable")
    sample = sorted(set([int(order[0]), int(order[-1]), 0, 255, 17, 128, 200]))
    for e in sample:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        ref, _ = OF.expert_forward(o["x"][src[lo:hi]], host(ex["w13"][e]), host(ex["w2"][e]))
        err = rel_max_err(host(yp[lo:hi]), ref)
        print(f"  expert {e} rows {hi - lo} rel max err {err:.3e}")
        assert err <= 2e-2
    del ex
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ["bf16", "e4m3", "f32"])
@pytest.mark.parametrize("counts,x_rows", [([0, 1, 300, 257, 129], 700), ([0, 0, 0], 513), ([64, 200], 1)])
def test_extra_group_equals_separate_call(dtype, counts, x_rows):
    """The shared expert as the extra group of the routed call (moe_ffn_extra):
    the routed outputs and the extra group's h and y bit-identical to two
    separate calls (bf16 on the matrix cores: one launch per product holding
    both; the other paths: launches of its own), including a call with no
    routed rows."""
    dev = need_gpu()
    print(f"ffn extra group {dtype} {counts} + {x_rows}", flush=True)
    g = torch.Generator(device=dev).manual_seed(sum(counts) + x_rows)
    d, d_ff = (1024, 512) if dtype != "f32" else (320, 96)
    n = len(counts)
    off = dev_i32(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32), dev)
    rows = max(int(sum(counts)), 1)
    x = torch.randn((rows, d), generator=g, device=dev).to(torch.bfloat16)
    xs = torch.randn((x_rows, d), generator=g, device=dev).to(torch.bfloat16)
    w13 = 0.05 * torch.randn((n, 2 * d_ff, d), generator=g, device=dev)
    w2 = 0.05 * torch.randn((n, d, d_ff), generator=g, device=dev)
    s13 = 0.05 * torch.randn((1, 2 * d_ff, d), generator=g, device=dev)
    s2 = 0.05 * torch.randn((1, d, d_ff), generator=g, device=dev)
    sc = {}
    if dtype == "e4m3":
        x, sc["xp_scale"] = M.quantize_rows_e4m3(x)
        xs, sc["x_scale"] = M.quantize_rows_e4m3(xs)
        w13, sc["w13_scale"] = M.quantize_blocks_e4m3(w13)
        w2, sc["w2_scale"] = M.quantize_blocks_e4m3(w2)
        s13, sc["s13"] = M.quantize_blocks_e4m3(s13)
        s2, sc["s2"] = M.quantize_blocks_e4m3(s2)
        dt = M.MOE_E4M3
    else:
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        x, xs, w13, w2, s13, s2 = (t.to(tdt) for t in (x, xs, w13, w2, s13, s2))
        dt = M.MOE_BF16 if dtype == "bf16" else M.MOE_F32
    # reference: two separate calls
    ref_y, ref_h, ref_hs = M.expert_ffn(off, rows, x, w13, w2, dt, xp_scale=sc.get("xp_scale"),
                                        w13_scale=sc.get("w13_scale"), w2_scale=sc.get("w2_scale"))
    ref_ys, ref_hx, ref_hxs = M.expert_ffn(dev_i32([0, x_rows], dev), x_rows, xs, s13, s2, dt,
                                           xp_scale=sc.get("x_scale"), w13_scale=sc.get("s13"),
                                           w2_scale=sc.get("s2"))
    # one call with the extra group
    store = {M.MOE_E4M3: torch.uint8, M.MOE_BF16: torch.bfloat16, M.MOE_F32: torch.float32}[dt]
    ydt = torch.float32 if dt == M.MOE_F32 else torch.bfloat16
    ex = dict(rows=x_rows, x=xs, x_scale=sc.get("x_scale"), w13=s13[0], w13_scale=sc.get("s13"), w2=s2[0],
              w2_scale=sc.get("s2"), h=torch.empty((x_rows, d_ff), dtype=store, device=dev),
              h_scale=(torch.empty((d_ff // 128, x_rows), dtype=torch.float32, device=dev)
                       if dt == M.MOE_E4M3 else None),
              y=torch.empty((x_rows, d), dtype=ydt, device=dev))
    y, h, hs = M.expert_ffn(off, rows, x, w13, w2, dt, xp_scale=sc.get("xp_scale"), w13_scale=sc.get("w13_scale"),
                            w2_scale=sc.get("w2_scale"), extra=ex)
    torch.cuda.synchronize()
    r = int(sum(counts))
    assert torch.equal(y[:r], ref_y[:r]) and torch.equal(h[:r], ref_h[:r])
    assert torch.equal(ex["y"], ref_ys) and torch.equal(ex["h"], ref_hx)
    if dt == M.MOE_E4M3:
        assert torch.equal(ex["h_scale"], ref_hxs)


def test_layer_merged_shared_equals_separate():
    """MoELayer with the shared expert merged into the routed launches gives
    the same output, bit for bit, as with a call of its own."""
    dev = need_gpu()
    cfg = C.get("flash").with_(T=1024, d=1024, E=16, G=4, k=4, M=2, d_ff=512)
    inp = gen.make_router(cfg, device=dev)
    ex = gen.make_experts(cfg, device=dev)
    outs = []
    for merge in (True, False):
        layer = M.MoELayer(cfg.T, cfg.d, cfg.E, cfg.G, cfg.M, cfg.k, cfg.d_ff, cfg.dtype, inp["w_gate"],
                           inp["bias"], ex["w13"], ex["w2"], ex["sh_w13"], ex["sh_w2"], group_topk=cfg.gk,
                           merge_shared=merge)
        outs.append(layer.forward(inp["x"]).clone())
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
