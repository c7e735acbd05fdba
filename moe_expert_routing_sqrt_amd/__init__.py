"""MI355X (gfx950) MoE-layer forward: Python binding of libmoe_mi355x.so.

The functions here only marshal torch tensors (device memory) and the current
HIP stream into the C ABI declared in include/moe.h; every step of the layer
runs in the library's HIP kernels.  There is no CPU or PyTorch fallback: if the
library is missing, or a tensor is not on the GPU, calls raise.

    route(shape, x, w_gate, bias)            -> logits, topk_idx, topk_w, block_counts
    route_hash(shape, token_ids, seed)       -> topk_idx, topk_w, block_counts
    dispatch(shape, topk_idx, block_counts, x) -> counts, offsets, dest, src, xp, xp_scale
    dispatch_noalloc(...)                    the same, its workspace in the library's static scratch
    expert_ffn(offsets, max_rows, xp, w13, w2) -> yp
    combine(shape, dest, topk_w, yp, ysh)    -> out
    bias_update(block_counts, bias, gamma)   -> load (bias updated in place)
    combine_backward / expert_ffn_backward / dispatch_backward / route_backward
                                             the layer's backward, stage by stage
    MoELayer                                 weights + buffers, forward(x) = the four calls
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib
from ._lib import (MOE_BF16, MOE_BWD_AU_SAVED, MOE_E4M3, MOE_F32, MOE_FFN_ALL, MOE_FFN_DOWN,  # noqa: F401
                   MOE_FFN_UP, MOE_FP8_TILE, MOE_OP_COMBINE, MOE_OP_DISPATCH, MOE_OP_EXPERT_FFN,
                   MOE_OP_EXPERT_FFN_BACKWARD, MOE_OP_ROUTE, MOE_OP_ROUTE_BACKWARD, MOE_ROUTE_BLOCK,
                   MOE_ROUTE_LOGITS_IN, MoeError, MoeFfnExtra, MoeShape)

__all__ = ["shape", "workspace_bytes", "workspace", "route", "route_hash", "dispatch", "dispatch_noalloc",
           "combine_backward",
           "expert_ffn_train",
           "expert_ffn_backward", "dispatch_backward", "route_backward", "expert_ffn", "combine",
           "quantize_blocks_e4m3", "quantize_rows_e4m3", "bias_update", "MoELayer", "MoeError", "lib"]


def lib():
    return _lib.load()


_DT = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16, torch.uint8: MOE_E4M3,
       torch.float8_e4m3fn: MOE_E4M3}
_TORCH = {MOE_F32: torch.float32, MOE_BF16: torch.bfloat16, MOE_E4M3: torch.uint8}


def _dt(t: torch.Tensor) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported tensor dtype {t.dtype}") from None


def _ptr(t: Optional[torch.Tensor]) -> int:
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError("tensors passed to the MoE library must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MoE library must be contiguous")
    return t.data_ptr()


def _stream(device=None) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need(t: Optional[torch.Tensor], numel: int, name: str):
    if t is not None and t.numel() < numel:
        raise ValueError(f"{name}: needs at least {numel} elements, has {t.numel()}")


def shape(T, d, E, G, M, k, d_ff, group_topk=None) -> MoeShape:
    gk = -(-k // M) if group_topk is None else group_topk
    return MoeShape(int(T), int(d), int(E), int(G), int(M), int(k), int(gk), int(d_ff))


def n_blocks(T: int) -> int:
    return (T + MOE_ROUTE_BLOCK - 1) // MOE_ROUTE_BLOCK


def workspace_bytes(op: int, sh: Optional[MoeShape] = None, dtype: int = MOE_BF16) -> int:
    """moe_workspace_size: device bytes a call of kind `op` (MOE_OP_*) needs."""
    if sh is None:
        sh = MoeShape(1, 1, 1, 1, 1, 1, 1, 1)
    return int(lib().moe_workspace_size(op, ctypes.byref(sh), dtype))


def workspace(op: int, sh: Optional[MoeShape], dtype: int, device) -> Optional[torch.Tensor]:
    """A zero-filled workspace for `op` (the expert products' ticket counters
    must start at zero), or None when the call needs none."""
    n = workspace_bytes(op, sh, dtype)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n > 0 else None


def _ws_len(ws: Optional[torch.Tensor]) -> int:
    return 0 if ws is None else ws.numel() * ws.element_size()


def route(sh: MoeShape, x: Optional[torch.Tensor], w_gate: Optional[torch.Tensor], bias: torch.Tensor,
          logit_offset: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None,
          logits_in: bool = False, idx=None, w=None, block_counts=None, ws: Optional[torch.Tensor] = None,
          keep_logits: bool = True):
    """Gate logits (fp32 W_g [d, E]), sqrt(softplus) affinities, node-limited
    top-k and block histogram.  keep_logits=False leaves the logits in the
    workspace (returned logits is then None)."""
    T, E, k = sh.T, sh.E, sh.k
    dev = bias.device
    if logits is None:
        if logits_in:
            raise ValueError("logits_in needs logits")
        if keep_logits:
            logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev) if idx is None else idx
    w = torch.empty((T, k), dtype=torch.float32, device=dev) if w is None else w
    if block_counts is None:
        block_counts = torch.empty((n_blocks(T), E), dtype=torch.int32, device=dev)
    _need(logits, T * E, "logits")
    _need(idx, T * k, "topk_idx")
    _need(w, T * k, "topk_w")
    _need(block_counts, n_blocks(T) * E, "block_counts")
    _need(bias, E, "bias")
    _need(logit_offset, E, "logit_offset")
    x_dtype = MOE_BF16
    if not logits_in:
        _need(x, T * sh.d, "x")
        _need(w_gate, sh.d * E, "w_gate")
        if w_gate.dtype != torch.float32:
            raise TypeError("w_gate must be fp32")
        x_dtype = _dt(x)
        if ws is None:
            ws = workspace(MOE_OP_ROUTE, sh, x_dtype, dev)
    st = lib().moe_route(ctypes.byref(sh), _ptr(x) if not logits_in else 0, x_dtype,
                         _ptr(w_gate) if not logits_in else 0, _ptr(bias), _ptr(logit_offset),
                         _ptr(logits), _ptr(idx), _ptr(w), _ptr(block_counts),
                         MOE_ROUTE_LOGITS_IN if logits_in else 0, _ptr(ws) if not logits_in else 0,
                         _ws_len(ws) if not logits_in else 0, _stream())
    _lib.check("moe_route", st)
    return logits, idx, w, block_counts


def route_hash(sh: MoeShape, token_ids: torch.Tensor, seed: int, logits: Optional[torch.Tensor] = None,
               idx=None, w=None, block_counts=None):
    """Hash router: each token's k experts from a Philox hash of its token id
    (int32 [T]); weights 1/k, or the renormalised affinities of those experts
    when logits [T, E] are given."""
    T, E, k = sh.T, sh.E, sh.k
    dev = token_ids.device
    if token_ids.dtype != torch.int32:
        raise TypeError("token_ids must be int32")
    idx = torch.empty((T, k), dtype=torch.int32, device=dev) if idx is None else idx
    w = torch.empty((T, k), dtype=torch.float32, device=dev) if w is None else w
    if block_counts is None:
        block_counts = torch.empty((n_blocks(T), E), dtype=torch.int32, device=dev)
    _need(token_ids, T, "token_ids")
    _need(idx, T * k, "topk_idx")
    _need(w, T * k, "topk_w")
    _need(block_counts, n_blocks(T) * E, "block_counts")
    _need(logits, T * E, "logits")
    st = lib().moe_route_hash(ctypes.byref(sh), _ptr(token_ids), int(seed) & ((1 << 64) - 1), _ptr(logits),
                              _ptr(idx), _ptr(w), _ptr(block_counts), _stream())
    _lib.check("moe_route_hash", st)
    return idx, w, block_counts


def dispatch(sh: MoeShape, idx: torch.Tensor, block_counts: torch.Tensor, x: torch.Tensor,
             e_begin: int = 0, e_end: Optional[int] = None, out_dtype: Optional[int] = None,
             bufs: Optional[dict] = None) -> dict:
    e_end = sh.E if e_end is None else e_end
    n = e_end - e_begin
    T, k, d = sh.T, sh.k, sh.d
    dev = x.device
    x_dtype = _dt(x)
    out_dtype = x_dtype if out_dtype is None else out_dtype
    b = {} if bufs is None else bufs
    rows = T * k
    if "counts" not in b:
        b["counts"] = torch.empty(n, dtype=torch.int32, device=dev)
        b["offsets"] = torch.empty(n + 1, dtype=torch.int32, device=dev)
        b["dest"] = torch.empty((T, k), dtype=torch.int32, device=dev)
        b["src"] = torch.empty(rows, dtype=torch.int32, device=dev)
        b["xp"] = torch.empty((rows, d), dtype=_TORCH[out_dtype], device=dev)
        b["xp_scale"] = (torch.empty((d // MOE_FP8_TILE, rows), dtype=torch.float32, device=dev)
                         if out_dtype == MOE_E4M3 else None)
        wsb = workspace_bytes(MOE_OP_DISPATCH, sh, out_dtype)
        b["ws"] = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    _need(b["counts"], n, "counts")
    _need(b["offsets"], n + 1, "offsets")
    _need(b["dest"], T * k, "dest")
    _need(b["src"], rows, "src")
    _need(b["xp"], rows * d, "xp")
    _need(x, T * d, "x")
    _need(idx, T * k, "topk_idx")
    _need(block_counts, n_blocks(T) * sh.E, "block_counts")
    if out_dtype == MOE_E4M3:
        _need(b["xp_scale"], rows * (d // MOE_FP8_TILE), "xp_scale")
    st = lib().moe_dispatch(ctypes.byref(sh), _ptr(idx), _ptr(block_counts), e_begin, e_end, _ptr(x),
                            x_dtype, out_dtype, _ptr(b["counts"]), _ptr(b["offsets"]), _ptr(b["dest"]),
                            _ptr(b["src"]), _ptr(b["xp"]), _ptr(b["xp_scale"]), _ptr(b["ws"]),
                            b["ws"].numel(), _stream())
    _lib.check("moe_dispatch", st)
    return b


def dispatch_noalloc(sh: MoeShape, idx: torch.Tensor, block_counts: torch.Tensor, x: torch.Tensor,
                     bufs: dict, e_begin: int = 0, e_end: Optional[int] = None,
                     out_dtype: Optional[int] = None) -> dict:
    """moe_dispatch_noalloc into caller-given output buffers (`bufs` with
    counts, offsets, dest, src, xp and, for e4m3, xp_scale, as dispatch()
    returns them): the call allocates nothing, its workspace is the library's
    static scratch."""
    e_end = sh.E if e_end is None else e_end
    n = e_end - e_begin
    T, k, d = sh.T, sh.k, sh.d
    x_dtype = _dt(x)
    out_dtype = x_dtype if out_dtype is None else out_dtype
    b = bufs
    _need(b["counts"], n, "counts")
    _need(b["offsets"], n + 1, "offsets")
    _need(b["dest"], T * k, "dest")
    _need(b["src"], T * k, "src")
    _need(b["xp"], T * k * d, "xp")
    _need(x, T * d, "x")
    _need(idx, T * k, "topk_idx")
    _need(block_counts, n_blocks(T) * sh.E, "block_counts")
    xs = b.get("xp_scale") if out_dtype == MOE_E4M3 else None
    if out_dtype == MOE_E4M3:
        _need(xs, T * k * (d // MOE_FP8_TILE), "xp_scale")
    st = lib().moe_dispatch_noalloc(ctypes.byref(sh), _ptr(idx), _ptr(block_counts), e_begin, e_end, _ptr(x),
                                    x_dtype, out_dtype, _ptr(b["counts"]), _ptr(b["offsets"]), _ptr(b["dest"]),
                                    _ptr(b["src"]), _ptr(b["xp"]), _ptr(xs), _stream())
    _lib.check("moe_dispatch_noalloc", st)
    return b


def expert_ffn(offsets: torch.Tensor, max_rows: int, xp: Optional[torch.Tensor], w13, w2,
               dtype: Optional[int] = None, xp_scale=None, w13_scale=None, w2_scale=None,
               h: Optional[torch.Tensor] = None, h_scale=None, yp: Optional[torch.Tensor] = None,
               stages: int = MOE_FFN_ALL, d: Optional[int] = None, d_ff: Optional[int] = None,
               ws: Optional[torch.Tensor] = None, extra: Optional[dict] = None):
    """Grouped SwiGLU experts over rows [offsets[i], offsets[i+1]) of xp.
    ws: the call's ticket-counter workspace (workspace(MOE_OP_EXPERT_FFN, ...):
    zero-filled once, left zero by every call); a fresh one when None.
    extra: one more group with buffers of its own (the shared expert), a dict
    with rows, x, w13, w2, h, y (and x_scale, w13_scale, w2_scale, h_scale
    for e4m3): moe_ffn_extra."""
    n_exp = offsets.numel() - 1
    ref = w13 if w13 is not None else w2
    dtype = _dt(ref) if dtype is None else dtype
    if w13 is not None:
        d_ff = w13.shape[1] // 2
        d = w13.shape[2]
    else:
        d, d_ff = w2.shape[1], w2.shape[2]
    dev = offsets.device
    if h is None:
        h = torch.empty((max_rows, d_ff), dtype=_TORCH[dtype], device=dev)
    if dtype == MOE_E4M3 and h_scale is None:
        h_scale = torch.empty((d_ff // MOE_FP8_TILE, max_rows), dtype=torch.float32, device=dev)
    if yp is None and stages & MOE_FFN_DOWN:
        yp = torch.empty((max_rows, d), dtype=torch.float32 if dtype == MOE_F32 else torch.bfloat16,
                         device=dev)
    if stages & MOE_FFN_UP:
        _need(xp, max_rows * d, "xp")
        _need(w13, n_exp * 2 * d_ff * d, "w13")
    if stages & MOE_FFN_DOWN:
        _need(w2, n_exp * d * d_ff, "w2")
        _need(yp, max_rows * d, "yp")
    _need(h, max_rows * d_ff, "h")
    if ws is None:
        ws = workspace(MOE_OP_EXPERT_FFN, None, dtype, dev)
    ex = None
    if extra is not None:
        r = int(extra["rows"])
        if stages & MOE_FFN_UP:
            _need(extra["x"], r * d, "extra x")
        if stages & MOE_FFN_DOWN:
            _need(extra["y"], r * d, "extra y")
        _need(extra["h"], r * d_ff, "extra h")
        ex = MoeFfnExtra(r, *[_ptr(extra.get(k)) for k in ("x", "x_scale", "w13", "w13_scale", "w2", "w2_scale",
                                                              "h", "h_scale", "y")])
    st = lib().moe_expert_ffn(n_exp, _ptr(offsets), max_rows, d, d_ff, dtype, _ptr(xp), _ptr(xp_scale),
                              _ptr(w13), _ptr(w13_scale), _ptr(w2), _ptr(w2_scale), _ptr(h),
                              _ptr(h_scale), _ptr(yp), stages, None if ex is None else ctypes.byref(ex),
                              _ptr(ws), _ws_len(ws), _stream())
    _lib.check("moe_expert_ffn", st)
    return yp, h, h_scale


def combine(sh: MoeShape, dest: torch.Tensor, topk_w: torch.Tensor, yp: torch.Tensor,
            ysh: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
            out_dtype: Optional[int] = None, accumulate: bool = False) -> torch.Tensor:
    T, d = sh.T, sh.d
    y_dtype = _dt(yp)
    if out is None:
        out_dtype = y_dtype if out_dtype is None else out_dtype
        out = torch.empty((T, d), dtype=_TORCH[out_dtype], device=yp.device)
    out_dtype = _dt(out)
    _need(out, T * d, "out")
    _need(ysh, T * d, "ysh")
    _need(dest, T * sh.k, "dest")
    _need(topk_w, T * sh.k, "topk_w")
    st = lib().moe_combine(ctypes.byref(sh), _ptr(dest), _ptr(topk_w), _ptr(yp), y_dtype, _ptr(ysh),
                           _ptr(out), out_dtype, 1 if accumulate else 0, _stream())
    _lib.check("moe_combine", st)
    return out


def quantize_rows_e4m3(x: torch.Tensor, q=None, scale=None):
    """bf16 [rows, cols] -> e4m3 codes (uint8) + fp32 scales per 1x128 row tile,
    stored block-major: scale [cols/128, rows]."""
    rows, cols = x.shape
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bf16")
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty((cols // MOE_FP8_TILE, rows), dtype=torch.float32, device=x.device)
    _need(q, rows * cols, "q")
    _need(scale, rows * (cols // MOE_FP8_TILE), "scale")
    st = lib().moe_quantize_rows_e4m3(rows, cols, _ptr(x), _ptr(q), _ptr(scale), _stream())
    _lib.check("moe_quantize_rows_e4m3", st)
    return q, scale


def quantize_blocks_e4m3(w: torch.Tensor, q=None, scale=None):
    """fp32 [..., rows, cols] -> e4m3 codes (uint8) + fp32 128x128 block scales."""
    rows, cols = w.shape[-2], w.shape[-1]
    n = w.numel() // (rows * cols)
    if q is None:
        q = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    if scale is None:
        scale = torch.empty((*w.shape[:-2], rows // MOE_FP8_TILE, cols // MOE_FP8_TILE),
                            dtype=torch.float32, device=w.device)
    _need(q, w.numel(), "q")
    _need(scale, n * (rows // MOE_FP8_TILE) * (cols // MOE_FP8_TILE), "scale")
    st = lib().moe_quantize_blocks_e4m3(n, rows, cols, _ptr(w), _ptr(q), _ptr(scale), _stream())
    _lib.check("moe_quantize_blocks_e4m3", st)
    return q, scale


def combine_backward(sh: MoeShape, dest, topk_w, yp, grad_out, d_yp=None, d_w=None):
    """d_yp [rows, d] bf16 and d_topk_w [T, k] fp32 of the combine."""
    T, k, d = sh.T, sh.k, sh.d
    rows = yp.shape[0]
    if d_yp is None:
        d_yp = torch.empty((rows, d), dtype=torch.bfloat16, device=yp.device)
    if d_w is None:
        d_w = torch.empty((T, k), dtype=torch.float32, device=yp.device)
    if d_yp.dtype != torch.bfloat16 or d_w.dtype != torch.float32:
        raise TypeError("d_yp must be bf16 and d_w fp32")
    _need(dest, T * k, "dest")
    _need(topk_w, T * k, "topk_w")
    _need(grad_out, T * d, "grad_out")
    _need(d_w, T * k, "d_topk_w")
    st = lib().moe_combine_backward(ctypes.byref(sh), _ptr(dest), _ptr(topk_w), _ptr(yp), _dt(yp), _ptr(grad_out),
                                    _dt(grad_out), _ptr(d_yp), _ptr(d_w), _stream())
    _lib.check("moe_combine_backward", st)
    return d_yp, d_w


def _ffn_bwd_ws(b: dict, max_rows: int, n_exp: int, d: int, d_ff: int, dev):
    bf = torch.bfloat16
    if "au" not in b:
        b["au"] = torch.empty((max_rows, 2 * d_ff), dtype=bf, device=dev)
        b["h"] = torch.empty((max_rows, d_ff), dtype=bf, device=dev)
        b["d_au"] = torch.empty((max_rows, 2 * d_ff), dtype=bf, device=dev)
        b["d_xp"] = torch.empty((max_rows, d), dtype=bf, device=dev)
        b["dw13"] = torch.empty((n_exp, 2 * d_ff, d), dtype=torch.float32, device=dev)
        b["dw2"] = torch.empty((n_exp, d, d_ff), dtype=torch.float32, device=dev)
    if "tickets" not in b:
        b["tickets"] = workspace(MOE_OP_EXPERT_FFN, None, MOE_BF16, dev)
        b["tickets_bwd"] = workspace(MOE_OP_EXPERT_FFN_BACKWARD, None, MOE_BF16, dev)
    return b


def expert_ffn_train(offsets: Optional[torch.Tensor], max_rows: int, xp, w13, w2, h, yp, ws: dict):
    """Grouped SwiGLU forward (bf16) that also keeps [a | u] in ws["au"] for
    expert_ffn_backward(..., au_saved=True).  h and yp as expert_ffn."""
    n_exp = 1 if offsets is None else offsets.numel() - 1
    d_ff, d = w13.shape[-2] // 2, w13.shape[-1]
    _ffn_bwd_ws(ws, max_rows, n_exp, d, d_ff, xp.device)
    _need(xp, max_rows * d, "xp")
    _need(h, max_rows * d_ff, "h")
    _need(yp, max_rows * d, "yp")
    st = lib().moe_expert_ffn_train(n_exp, _ptr(offsets), max_rows, d, d_ff, _dt(xp), _ptr(xp), _ptr(w13), _ptr(w2),
                                    _ptr(h), _ptr(ws["au"]), _ptr(yp), _ptr(ws["tickets"]), _ws_len(ws["tickets"]),
                                    _stream())
    _lib.check("moe_expert_ffn_train", st)
    return yp, h


def expert_ffn_backward(offsets: Optional[torch.Tensor], max_rows: int, xp, w13, w2, d_yp, ws: Optional[dict] = None,
                        au_saved: bool = False):
    """Grouped SwiGLU backward: returns dict with d_xp [max_rows, d] bf16, dw13
    [n, 2*d_ff, d] fp32, dw2 [n, d, d_ff] fp32 (and the bf16 workspaces).
    au_saved: ws["au"] holds expert_ffn_train's [a | u] (no recompute)."""
    n_exp = 1 if offsets is None else offsets.numel() - 1
    d_ff, d = w13.shape[-2] // 2, w13.shape[-1]
    dev = xp.device
    b = {} if ws is None else ws
    if au_saved and "au" not in b:
        raise ValueError("au_saved needs ws['au'] from expert_ffn_train")
    _ffn_bwd_ws(b, max_rows, n_exp, d, d_ff, dev)
    _need(xp, max_rows * d, "xp")
    _need(d_yp, max_rows * d, "d_yp")
    _need(w13, n_exp * 2 * d_ff * d, "w13")
    _need(w2, n_exp * d * d_ff, "w2")
    for n, need in (("au", max_rows * 2 * d_ff), ("h", max_rows * d_ff), ("d_au", max_rows * 2 * d_ff),
                    ("d_xp", max_rows * d), ("dw13", n_exp * 2 * d_ff * d), ("dw2", n_exp * d * d_ff)):
        _need(b[n], need, n)
    st = lib().moe_expert_ffn_backward(n_exp, _ptr(offsets), max_rows, d, d_ff, _dt(xp), _ptr(xp), _ptr(w13),
                                       _ptr(w2), _ptr(d_yp), _ptr(b["au"]), _ptr(b["h"]), _ptr(b["d_au"]),
                                       _ptr(b["d_xp"]), _ptr(b["dw13"]), _ptr(b["dw2"]),
                                       MOE_BWD_AU_SAVED if au_saved else 0, _ptr(b["tickets_bwd"]),
                                       _ws_len(b["tickets_bwd"]), _stream())
    _lib.check("moe_expert_ffn_backward", st)
    return b


def dispatch_backward(sh: MoeShape, dest, d_xp, d_extra=None, dx=None, accumulate: bool = False):
    """dx [T, d] fp32 (+)= d_extra + sum_j d_xp[dest[t, j]]."""
    T, d = sh.T, sh.d
    if dx is None:
        dx = torch.empty((T, d), dtype=torch.float32, device=d_xp.device)
    if dx.dtype != torch.float32:
        raise TypeError("dx must be fp32")
    if d_extra is not None and d_extra.dtype != d_xp.dtype:
        raise TypeError("d_extra must have d_xp's dtype")
    _need(dest, T * sh.k, "dest")
    _need(d_extra, T * d, "d_extra")
    _need(dx, T * d, "dx")
    st = lib().moe_dispatch_backward(ctypes.byref(sh), _ptr(dest), _ptr(d_xp), _dt(d_xp), _ptr(d_extra), _ptr(dx),
                                     1 if accumulate else 0, _stream())
    _lib.check("moe_dispatch_backward", st)
    return dx


def route_backward(sh: MoeShape, x, w_gate, logits, idx, d_w, dx, logit_offset=None, dlogits=None,
                   dw_gate=None, ws=None):
    """Gate path: dlogits [T, E] (written), dx += dlogits W_g^T, dw_gate = x^T dlogits."""
    T, E, d = sh.T, sh.E, sh.d
    dev = x.device
    if dlogits is None:
        dlogits = torch.empty((T, E), dtype=torch.float32, device=dev)
    if dw_gate is None:
        dw_gate = torch.empty((d, E), dtype=torch.float32, device=dev)
    if w_gate.dtype != torch.float32 or dx.dtype != torch.float32:
        raise TypeError("w_gate and dx must be fp32")
    _need(x, T * d, "x")
    _need(w_gate, d * E, "w_gate")
    _need(logits, T * E, "logits")
    _need(idx, T * sh.k, "topk_idx")
    _need(d_w, T * sh.k, "d_topk_w")
    _need(dlogits, T * E, "dlogits")
    _need(dx, T * d, "dx")
    _need(dw_gate, d * E, "dw_gate")
    _need(logit_offset, E, "logit_offset")
    wsb = workspace_bytes(MOE_OP_ROUTE_BACKWARD, sh, _dt(x))
    if ws is None and wsb > 0:
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    st = lib().moe_route_backward(ctypes.byref(sh), _ptr(x), _dt(x), _ptr(w_gate), _ptr(logit_offset), _ptr(logits),
                                  _ptr(idx), _ptr(d_w), _ptr(dlogits), _ptr(dx), _ptr(dw_gate), _ptr(ws),
                                  _ws_len(ws), _stream())
    _lib.check("moe_route_backward", st)
    return dlogits, dw_gate


def bias_update(counts: torch.Tensor, bias: torch.Tensor, gamma: float,
                load: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bias[e] += gamma * sign(mean load - load[e]) in place, with load[e] the
    column sums of counts [n_rows, E] (moe_route's block counts, or one load
    vector).  Returns load [E] int32 (allocated when not given)."""
    E = bias.numel()
    if bias.dtype != torch.float32 or counts.dtype != torch.int32:
        raise TypeError("bias must be float32 and counts int32")
    if not (bias.is_contiguous() and counts.is_contiguous()):
        raise ValueError("bias and counts must be contiguous")
    n_rows = counts.numel() // E if E else 0
    if load is None:
        load = torch.empty(E, dtype=torch.int32, device=bias.device)
    _need(counts, n_rows * E, "counts")
    _need(load, E, "load")
    st = lib().moe_bias_update(n_rows, E, _ptr(counts), float(gamma), _ptr(bias), _ptr(load), _stream())
    _lib.check("moe_bias_update", st)
    return load


from .layer import MoELayer  # noqa: E402
