"""MoELayer: one MoE layer forward on one GPU, weights resident and every
buffer allocated once, so forward() only enqueues the library's kernels.

forward(x) = moe_route -> moe_dispatch -> moe_expert_ffn (routed: up, down)
             -> moe_expert_ffn (shared expert) -> moe_combine
"""
from __future__ import annotations

from typing import Optional, Sequence

import torch

from . import (MOE_BF16, MOE_E4M3, MOE_F32, MOE_FFN_ALL, MOE_FFN_DOWN, MOE_FFN_UP, MOE_FP8_TILE,
               MOE_OP_EXPERT_FFN, MOE_OP_ROUTE, MOE_OP_ROUTE_BACKWARD, bias_update, combine, combine_backward,
               dispatch, dispatch_backward, expert_ffn, expert_ffn_backward, expert_ffn_train, n_blocks,
               quantize_blocks_e4m3, quantize_rows_e4m3, route, route_backward, route_hash, shape,
               workspace, workspace_bytes)

STAGES = ("route", "dispatch", "ffn_up", "ffn_down", "shared", "combine")


class MoELayer:
    def __init__(self, T: int, d: int, E: int, G: int, M: int, k: int, d_ff: int, dtype: str,
                 w_gate: torch.Tensor, bias: torch.Tensor, w13: torch.Tensor, w2: torch.Tensor,
                 sh_w13: Optional[torch.Tensor] = None, sh_w2: Optional[torch.Tensor] = None,
                 logit_offset: Optional[torch.Tensor] = None, e_begin: int = 0,
                 e_end: Optional[int] = None, group_topk: Optional[int] = None,
                 router: str = "topk", hash_seed: int = 0, merge_shared: bool = True):
        dev = bias.device
        self.sh = shape(T, d, E, G, M, k, d_ff, group_topk)
        self.T, self.d, self.E, self.k, self.d_ff = T, d, E, k, d_ff
        self.e_begin, self.e_end = e_begin, (E if e_end is None else e_end)
        self.local = (self.e_begin, self.e_end) != (0, E)
        self.dtype = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_E4M3}[dtype]
        self.bias = bias
        self.w_gate = w_gate
        self.logit_offset = logit_offset
        if router not in ("topk", "hash"):
            raise ValueError("router must be 'topk' or 'hash'")
        self.router, self.hash_seed = router, hash_seed
        x_dt = MOE_F32 if dtype == "f32" else MOE_BF16
        # caller-owned workspaces, one per call site: the route's (gate-weight
        # planes), and the ticket counters of the routed and shared expert
        # products (zero-filled once; every call leaves them zero)
        self.route_ws = workspace(MOE_OP_ROUTE, self.sh, x_dt, dev)
        self.ffn_ws = workspace(MOE_OP_EXPERT_FFN, None, MOE_BF16, dev)
        self.sh_ffn_ws = workspace(MOE_OP_EXPERT_FFN, None, MOE_BF16, dev)

        # expert weights in the compute format (fp8: e4m3 codes + 128x128 block scales)
        if self.dtype == MOE_E4M3:
            self.w13, self.w13_s = quantize_blocks_e4m3(w13)
            self.w2, self.w2_s = quantize_blocks_e4m3(w2)
            if sh_w13 is not None:
                self.sh_w13, self.sh_w13_s = quantize_blocks_e4m3(sh_w13)
                self.sh_w2, self.sh_w2_s = quantize_blocks_e4m3(sh_w2)
        else:
            self.w13, self.w2, self.w13_s, self.w2_s = w13, w2, None, None
            self.sh_w13, self.sh_w2 = sh_w13, sh_w2
            self.sh_w13_s = self.sh_w2_s = None
        self.has_shared = sh_w13 is not None and not self.local
        # the shared expert as one more group of the routed expert launches
        # (moe_ffn_extra) where the library computes it inside them (bf16
        # matrix-core products); otherwise, or with merge_shared=False, a call
        # of its own after them
        mfma = self.dtype == MOE_BF16 and d % 256 == 0 and d_ff % 128 == 0 and d_ff >= 256
        self.merge_shared = merge_shared and self.has_shared and mfma

        act = torch.float32 if self.dtype == MOE_F32 else torch.bfloat16
        store = {MOE_F32: torch.float32, MOE_BF16: torch.bfloat16, MOE_E4M3: torch.uint8}[self.dtype]
        rows = T * k
        self.max_rows = rows
        self.logits = torch.empty((T, E), dtype=torch.float32, device=dev)
        self.idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.block_counts = torch.empty((n_blocks(T), E), dtype=torch.int32, device=dev)
        self.dbufs = None
        self.h = torch.empty((rows, d_ff), dtype=store, device=dev)
        self.h_s = (torch.empty((d_ff // MOE_FP8_TILE, rows), dtype=torch.float32, device=dev)
                    if self.dtype == MOE_E4M3 else None)
        self.yp = torch.empty((rows, d), dtype=act, device=dev)
        if self.has_shared:
            self.sh_offsets = torch.tensor([0, T], dtype=torch.int32, device=dev)
            self.sh_h = torch.empty((T, d_ff), dtype=store, device=dev)
            self.sh_h_s = (torch.empty((d_ff // MOE_FP8_TILE, T), dtype=torch.float32, device=dev)
                           if self.dtype == MOE_E4M3 else None)
            self.ysh = torch.empty((T, d), dtype=act, device=dev)
            if self.dtype == MOE_E4M3:
                self.sh_xq = torch.empty((T, d), dtype=torch.uint8, device=dev)
                self.sh_xs = torch.empty((d // MOE_FP8_TILE, T), dtype=torch.float32, device=dev)
        self.out = torch.empty((T, d), dtype=torch.float32 if self.local else act, device=dev)

    def update_bias(self, gamma: float) -> torch.Tensor:
        """Auxiliary-loss-free balancing step after a forward: moves each
        expert's routing bias by gamma towards the mean load of the last
        batch (moe_bias_update on the route's block counts).  Returns the
        per-expert load [E]."""
        if not hasattr(self, "load"):
            self.load = torch.empty(self.E, dtype=torch.int32, device=self.bias.device)
        return bias_update(self.block_counts, self.bias, gamma, self.load)

    def forward(self, x: torch.Tensor, out: Optional[torch.Tensor] = None,
                marks: Optional[Sequence[torch.cuda.Event]] = None,
                token_ids: Optional[torch.Tensor] = None, save_for_backward: bool = False) -> torch.Tensor:
        """One layer forward.  `marks`: optional 7 events recorded on the current
        stream around the six stages (STAGES).  With router="hash" the experts
        come from `token_ids` (int32 [T]) and the gate weights are 1/k.
        save_for_backward: the expert FFNs also keep their pre-activations, so
        backward() does not recompute them (bf16 top-k layer).
        With a local expert range (one expert-parallel rank's share) the
        output is that share in fp32: written to self.out (0 for tokens with no
        local expert) when `out` is None, else added to the caller's fp32 `out`
        (a scatter-add of this rank's share into a buffer that may hold the
        others')."""
        self._saved = save_for_backward
        if save_for_backward:
            return self._forward_train(x, marks)
        def mark(i):
            if marks is not None:
                marks[i].record()

        sh = self.sh
        mark(0)
        if self.router == "hash":
            if token_ids is None:
                raise ValueError("the hash router needs token_ids")
            route_hash(sh, token_ids, self.hash_seed, idx=self.idx, w=self.topk_w,
                       block_counts=self.block_counts)
        else:
            route(sh, x, self.w_gate, self.bias, self.logit_offset, logits=self.logits, idx=self.idx,
                  w=self.topk_w, block_counts=self.block_counts, ws=self.route_ws)
        mark(1)
        self.dbufs = dispatch(sh, self.idx, self.block_counts, x, self.e_begin, self.e_end,
                              out_dtype=self.dtype if self.dtype == MOE_E4M3 else None,
                              bufs=self.dbufs)
        b = self.dbufs
        mark(2)
        extra = None
        if self.merge_shared:
            extra = dict(rows=self.T, x=x, w13=self.sh_w13, w2=self.sh_w2, h=self.sh_h, y=self.ysh)
        expert_ffn(b["offsets"], self.max_rows, b["xp"], self.w13, self.w2, self.dtype,
                   xp_scale=b["xp_scale"], w13_scale=self.w13_s, w2_scale=self.w2_s, h=self.h,
                   h_scale=self.h_s, yp=self.yp, stages=MOE_FFN_UP, ws=self.ffn_ws, extra=extra)
        mark(3)
        expert_ffn(b["offsets"], self.max_rows, b["xp"], self.w13, self.w2, self.dtype,
                   xp_scale=b["xp_scale"], w13_scale=self.w13_s, w2_scale=self.w2_s, h=self.h,
                   h_scale=self.h_s, yp=self.yp, stages=MOE_FFN_DOWN, ws=self.ffn_ws, extra=extra)
        mark(4)
        ysh = self.ysh if self.merge_shared else None
        if self.has_shared and not self.merge_shared:
            xs, xs_scale = x, None
            if self.dtype == MOE_E4M3:
                xs, xs_scale = self._shared_quant_input(x)
            expert_ffn(self.sh_offsets, self.T, xs, self.sh_w13, self.sh_w2, self.dtype,
                       xp_scale=xs_scale, w13_scale=self.sh_w13_s, w2_scale=self.sh_w2_s,
                       h=self.sh_h, h_scale=self.sh_h_s, yp=self.ysh, stages=MOE_FFN_ALL, ws=self.sh_ffn_ws)
            ysh = self.ysh
        mark(5)
        if out is None:
            # the layer's own output: every row written (a local share's rows
            # without a local expert get 0), nothing read back
            combine(sh, b["dest"], self.topk_w, self.yp, ysh, out=self.out, accumulate=False)
            out = self.out
        else:
            combine(sh, b["dest"], self.topk_w, self.yp, ysh, out=out, accumulate=self.local)
        mark(6)
        return out

    def _bwd_ws(self, dev):
        if not hasattr(self, "bws"):
            self.bws = {"routed": {}, "shared": {},
                        "d_yp": torch.empty((self.max_rows, self.d), dtype=torch.bfloat16, device=dev),
                        "d_w": torch.empty((self.T, self.k), dtype=torch.float32, device=dev),
                        "dx": torch.empty((self.T, self.d), dtype=torch.float32, device=dev),
                        "dlogits": torch.empty((self.T, self.E), dtype=torch.float32, device=dev),
                        "dw_gate": torch.empty((self.d, self.E), dtype=torch.float32, device=dev)}
            wsb = workspace_bytes(MOE_OP_ROUTE_BACKWARD, self.sh, MOE_BF16)
            self.bws["gate_ws"] = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
        return self.bws

    def _forward_train(self, x, marks):
        if self.dtype != MOE_BF16 or self.local or self.router != "topk":
            raise ValueError("save_for_backward covers the bf16 top-k layer with all experts local")

        def mark(i):
            if marks is not None:
                marks[i].record()

        sh, w = self.sh, self._bwd_ws(x.device)
        mark(0)
        route(sh, x, self.w_gate, self.bias, self.logit_offset, logits=self.logits, idx=self.idx,
              w=self.topk_w, block_counts=self.block_counts, ws=self.route_ws)
        mark(1)
        self.dbufs = dispatch(sh, self.idx, self.block_counts, x, self.e_begin, self.e_end, bufs=self.dbufs)
        b = self.dbufs
        mark(2)
        expert_ffn_train(b["offsets"], self.max_rows, b["xp"], self.w13, self.w2, self.h, self.yp, w["routed"])
        mark(3)
        mark(4)
        ysh = None
        if self.has_shared:
            expert_ffn_train(None, self.T, x, self.sh_w13, self.sh_w2, self.sh_h, self.ysh, w["shared"])
            ysh = self.ysh
        mark(5)
        combine(sh, b["dest"], self.topk_w, self.yp, ysh, out=self.out)
        mark(6)
        return self.out

    def backward(self, x: torch.Tensor, grad_out: torch.Tensor,
                 marks: Optional[Sequence[torch.cuda.Event]] = None) -> dict:
        """Gradients of the last forward(x) for grad_out = d loss / d out (bf16
        [T, d]): dx [T, d] fp32, dw_gate [d, E] fp32, dw13 / dw2 of the routed
        experts and dsh_w13 / dsh_w2 of the shared expert (fp32).  The expert
        selection of the forward is held fixed; the routing bias gets no
        gradient.  `marks`: optional 5 events around the four stages
        (combine, routed experts, shared expert, dispatch + gate)."""
        if self.dtype != MOE_BF16 or self.local or self.router != "topk":
            raise ValueError("backward covers the bf16 top-k layer with all experts local")
        if grad_out.dtype != torch.bfloat16:
            raise TypeError("grad_out must be bf16")

        def mark(i):
            if marks is not None:
                marks[i].record()

        sh, b, dev = self.sh, self.dbufs, x.device
        w = self._bwd_ws(dev)
        saved = getattr(self, "_saved", False)
        mark(0)
        combine_backward(sh, b["dest"], self.topk_w, self.yp, grad_out, w["d_yp"], w["d_w"])
        mark(1)
        r = expert_ffn_backward(b["offsets"], self.max_rows, b["xp"], self.w13, self.w2, w["d_yp"], w["routed"],
                                au_saved=saved)
        mark(2)
        sx = None
        if self.has_shared:
            s_ = expert_ffn_backward(None, self.T, x, self.sh_w13, self.sh_w2, grad_out, w["shared"],
                                     au_saved=saved)
            sx = s_["d_xp"]
        mark(3)
        dispatch_backward(sh, b["dest"], r["d_xp"], d_extra=sx, dx=w["dx"])
        route_backward(sh, x, self.w_gate, self.logits, self.idx, w["d_w"], w["dx"],
                       logit_offset=self.logit_offset, dlogits=w["dlogits"], dw_gate=w["dw_gate"],
                       ws=w["gate_ws"])
        mark(4)
        out = {"dx": w["dx"], "dw_gate": w["dw_gate"], "dw13": r["dw13"], "dw2": r["dw2"],
               "d_topk_w": w["d_w"]}
        if self.has_shared:
            out["dsh_w13"], out["dsh_w2"] = w["shared"]["dw13"], w["shared"]["dw2"]
        return out

    def _shared_quant_input(self, x):
        return quantize_rows_e4m3(x, self.sh_xq, self.sh_xs)
