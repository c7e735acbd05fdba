"""GPU parity: combine (S5) against the oracle's fp64 combine."""
import numpy as np
import pytest
import torch

import moe_expert_routing_sqrt_amd as M
from moe_inputs import configs as C
from oracle import combine as OC, dispatch as OD

from gpu_util import dev_f32, dev_i32, host, moe_shape, need_gpu, rel_max_err, router_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny", "flash", "v3"])
def test_combine_workload(name):
    dev = need_gpu()
    cfg, inp, o = router_inputs(name)
    print(f"combine S5 {name}", flush=True)
    counts, offsets, dest, src = OD.dispatch(o["idx"], cfg.E)
    act = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    g = torch.Generator(device=dev).manual_seed(7)
    yp = torch.randn((cfg.pairs, cfg.d), generator=g, device=dev).to(act)
    ysh = torch.randn((cfg.T, cfg.d), generator=g, device=dev).to(act)
    out = M.combine(moe_shape(cfg), dev_i32(dest, dev), dev_f32(o["w"], dev), yp, ysh)
    torch.cuda.synchronize()
    ref = OC.combine(host(yp), dest, o["w"], ysh=host(ysh))
    err = rel_max_err(host(out), ref)
    print(f"  rel max err {err:.3e}")
    assert err <= (1e-6 if act == torch.float32 else 2e-2)
    if act == torch.bfloat16:
        # elementwise: one bf16 rounding of an fp32 sum
        assert np.all(np.abs(host(out) - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5 * np.abs(ref).max())


@pytest.mark.timeout(400)
def test_combine_max_size_sampled():
    """65536 tokens at V3 (524288 rows of 7168): 2048 sampled tokens and the
    last one against the oracle's combine of just those tokens' rows."""
    dev = need_gpu()
    cfg, inp, o = router_inputs("v3", 65536)
    print(f"combine S5 v3 T={cfg.T} (sampled tokens)", flush=True)
    counts, offsets, dest, src = OD.dispatch(o["idx"], cfg.E)
    g = torch.Generator(device=dev).manual_seed(17)
    yp = torch.randn((cfg.pairs, cfg.d), generator=g, device=dev).to(torch.bfloat16)
    ysh = torch.randn((cfg.T, cfg.d), generator=g, device=dev).to(torch.bfloat16)
    out = M.combine(moe_shape(cfg), dev_i32(dest, dev), dev_f32(o["w"], dev), yp, ysh)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    toks = np.array(sorted(set(rng.choice(cfg.T, 2048, replace=False).tolist()) | {cfg.T - 1}))
    rows = dest[toks].reshape(-1)
    tdev = torch.from_numpy(toks.astype(np.int64)).to(dev)
    yp_sub = host(yp[torch.from_numpy(rows.astype(np.int64)).to(dev)])
    dest_sub = np.arange(rows.size, dtype=np.int32).reshape(len(toks), cfg.k)
    ref = OC.combine(yp_sub, dest_sub, o["w"][toks], ysh=host(ysh[tdev]))
    got = host(out[tdev])
    err = rel_max_err(got, ref)
    print(f"  rel max err {err:.3e} on {len(toks)} tokens")
    assert err <= 2e-2
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5 * np.abs(ref).max())


def test_identity_experts_give_weight_sum_times_x():
    dev = need_gpu()
    cfg, inp, o = router_inputs("flash")
    counts, offsets, dest, src = OD.dispatch(o["idx"], cfg.E)
    xp = inp["x"][torch.from_numpy(src.astype(np.int64)).to(dev)].contiguous().float()
    out = M.combine(moe_shape(cfg), dev_i32(dest, dev), dev_f32(o["w"], dev), xp, None,
                    out_dtype=M.MOE_F32)
    torch.cuda.synchronize()
    expect = o["w"].astype(np.float64).sum(1, keepdims=True) * o["x"]
    assert np.allclose(host(out), expect, rtol=2e-6, atol=1e-6)


def test_accumulate_local_share():
    dev = need_gpu()
    cfg, inp, o = router_inputs("v3_skew_ep0")
    counts, offsets, dest, src = OD.dispatch(o["idx"], cfg.E, 0, 4)
    rows = int(offsets[-1])
    g = torch.Generator(device=dev).manual_seed(9)
    yp = torch.randn((max(rows, 1), cfg.d), generator=g, device=dev).to(torch.bfloat16)
    init = torch.randn((cfg.T, cfg.d), generator=g, device=dev)
    out = init.clone()
    M.combine(moe_shape(cfg), dev_i32(dest, dev), dev_f32(o["w"], dev), yp, None, out=out, accumulate=True)
    torch.cuda.synchronize()
    ref = OC.combine(host(yp), dest, o["w"], out_init=host(init))
    assert rel_max_err(host(out), ref) <= 1e-6
    untouched = (dest < 0).all(1)
    assert np.array_equal(host(out)[untouched], host(init)[untouched])


def test_ragged_token_count():
    dev = need_gpu()
    cfg = C.FLASH.with_(T=7, d=128)
    rng = np.random.default_rng(1)
    idx = np.stack([rng.choice(cfg.E, cfg.k, replace=False) for _ in range(cfg.T)]).astype(np.int32)
    w = rng.random((cfg.T, cfg.k)).astype(np.float32)
    _, _, dest, _ = OD.dispatch(idx, cfg.E)
    yp = torch.randn((cfg.pairs, cfg.d), device=dev).to(torch.bfloat16)
    out = M.combine(moe_shape(cfg), dev_i32(dest, dev), dev_f32(w, dev), yp, None, out_dtype=M.MOE_F32)
    torch.cuda.synchronize()
    assert rel_max_err(host(out), OC.combine(host(yp), dest, w)) <= 1e-6
