"""GPU parity: dispatch from the oracle's routing (S3).  counts, offsets,
dest, src and the packed rows must match the oracle bit for bit."""
import numpy as np
import pytest
import torch

import moe_expert_routing_sqrt_amd as M
from moe_inputs import configs as C
from oracle import dispatch as OD

from gpu_util import block_counts, dev_i32, host, moe_shape, need_gpu, router_inputs

pytestmark = pytest.mark.gpu


def _run(cfg, x_dev, idx, e_begin=0, e_end=None, out_dtype=None):
    dev = x_dev.device
    sh = moe_shape(cfg)
    e_end = cfg.E if e_end is None else e_end
    b = M.dispatch(sh, dev_i32(idx, dev), dev_i32(block_counts(idx, cfg.E), dev), x_dev, e_begin, e_end,
                   out_dtype=out_dtype)
    torch.cuda.synchronize()
    return b


def _check(cfg, x_dev, x_h, idx, e_begin=0, e_end=None):
    e_end = cfg.E if e_end is None else e_end
    b = _run(cfg, x_dev, idx, e_begin, e_end)
    counts, offsets, dest, src = OD.dispatch(idx, cfg.E, e_begin, e_end)
    rows = int(offsets[-1])
    assert np.array_equal(host(b["counts"]), counts)
    assert np.array_equal(host(b["offsets"]), offsets)
    assert np.array_equal(host(b["dest"]), dest)
    assert np.array_equal(host(b["src"])[:rows], src)
    # packed rows: bitwise copies of x rows
    xp = b["xp"][:rows]
    ref = x_dev[torch.from_numpy(src.astype(np.int64)).to(x_dev.device)]
    assert torch.equal(xp.view(torch.int16) if xp.dtype == torch.bfloat16 else xp.view(torch.int32),
                       ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref.view(torch.int32))
    return b


@pytest.mark.timeout(400)
@pytest.mark.parametrize("name,T", [("tiny", None), ("flash", None), ("v3", None), ("v3", 1000), ("tiny", 63),
                                    ("flash", 1), ("v3", 65536)])
def test_dispatch_bitexact(name, T):
    """Up to 65536 tokens at V3 (524288 packed rows, 7.5 GB)."""
    dev = need_gpu()
    cfg, inp, o = router_inputs(name, T)
    print(f"dispatch S3 {name} T={cfg.T}", flush=True)
    _check(cfg, inp["x"], o["x"], o["idx"])


@pytest.mark.parametrize("eb,ee", [(0, 4), (252, 256), (100, 164), (0, 256)])
def test_dispatch_expert_range_skewed(eb, ee):
    dev = need_gpu()
    cfg, inp, o = router_inputs("v3_skew_ep0")
    print(f"dispatch range [{eb},{ee})", flush=True)
    b = _check(cfg, inp["x"], o["x"], o["idx"], eb, ee)
    c = host(b["counts"])
    if (eb, ee) == (0, 256):
        # the Zipf offset skews the load by an order of magnitude
        assert c.max() >= 10 * max(c.min(), 1)


def test_dispatch_hot_and_empty_experts():
    dev = need_gpu()
    cfg = C.FLASH.with_(T=777)
    rng = np.random.default_rng(3)
    idx = np.tile(np.arange(cfg.k, dtype=np.int32), (cfg.T, 1))      # every token -> experts 0..k-1
    idx[::5] = rng.permutation(cfg.E)[: cfg.k]                         # a few elsewhere
    x = torch.randn((cfg.T, cfg.d), device=dev).to(torch.bfloat16)
    _check(cfg, x, host(x), idx)


def test_dispatch_f32_rows():
    dev = need_gpu()
    cfg, inp, o = router_inputs("tiny")
    assert inp["x"].dtype == torch.float32
    _check(cfg, inp["x"], o["x"], o["idx"], 4, 12)


def test_dispatch_deterministic_repeat():
    dev = need_gpu()
    cfg, inp, o = router_inputs("v3")
    b1 = _run(cfg, inp["x"], o["idx"])
    snap = {k: v.clone() for k, v in b1.items() if v is not None and k != "ws"}
    b2 = _run(cfg, inp["x"], o["idx"])
    for k, v in snap.items():
        assert torch.equal(v, b2[k]), k
