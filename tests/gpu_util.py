"""Helpers for the GPU parity tests: device setup, host copies, metrics and
oracle-side derived values.  Expected values come only from oracle/ (run on the
host on the same seeded inputs); nothing here reads a GPU result back into an
expected value."""
import functools

import numpy as np
import pytest
import torch

from moe_inputs import configs as C, generate as gen
from oracle import dispatch as OD, ffn as OF, route as OR

ROUTE_BLOCK = 64


def need_gpu() -> torch.device:
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    return torch.device("cuda")


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


def rel_max_err(got, ref) -> float:
    """max |got - ref| / max |ref| over the whole tensor (the stated metric)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))


def logits_row_err(got, ref) -> float:
    """per row: max_e |dL| / max_e |L_ref|; returns the worst row."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float((np.abs(got - ref).max(1) / np.maximum(np.abs(ref).max(1), 1e-30)).max())


def block_counts(idx: np.ndarray, E: int) -> np.ndarray:
    T = idx.shape[0]
    nb = (T + ROUTE_BLOCK - 1) // ROUTE_BLOCK
    out = np.zeros((nb, E), dtype=np.int32)
    for b in range(nb):
        out[b] = np.bincount(idx[b * ROUTE_BLOCK:(b + 1) * ROUTE_BLOCK].ravel(), minlength=E)
    return out


def dev_i32(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


def dev_f32(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


@functools.lru_cache(maxsize=8)
def router_inputs(name: str, T: int = None):
    """Router inputs on the GPU (generated there) + host copies + the oracle's
    fp64-formed fp32 logits and routing."""
    dev = need_gpu()
    cfg = C.get(name)
    if T is not None:
        cfg = cfg.with_(T=T)
    inp = gen.make_router(cfg, device=dev)
    x_h = host(inp["x"])
    wg_h = host(inp["w_gate"])
    bias_h = host(inp["bias"])
    off_h = None if inp["logit_offset"] is None else host(inp["logit_offset"])
    L = OR.gate_logits(x_h, wg_h)
    idx, w = OR.route_from_logits(L, bias_h, cfg.G, cfg.M, cfg.k, cfg.gk, off_h)
    return cfg, inp, dict(x=x_h, w_gate=wg_h, bias=bias_h, offset=off_h, L=L, idx=idx, w=w)


def moe_shape(cfg):
    import moe_expert_routing_sqrt_amd as M
    return M.shape(cfg.T, cfg.d, cfg.E, cfg.G, cfg.M, cfg.k, cfg.d_ff, cfg.gk)


def expert_host(cfg, e, dev, shared=False):
    """fp32 host copies of one expert's weights as the GPU holds them."""
    w13, w2 = gen.expert_weights(cfg, e, device=dev, shared=shared)
    return host(w13), host(w2)


def cu_mask_stream(torch, words_mask):
    """A torch stream on a HIP stream limited to the CUs of a bit mask (one bit
    per CU, 32 per word: hipExtStreamCreateWithCUMask), default priority."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    h = ctypes.c_void_p()
    arr = (ctypes.c_uint32 * len(words_mask))(*words_mask)
    st = hip.hipExtStreamCreateWithCUMask(ctypes.byref(h), ctypes.c_uint32(len(words_mask)), arr)
    assert st == 0, f"hipExtStreamCreateWithCUMask failed ({st})"
    return torch.cuda.ExternalStream(h.value)
