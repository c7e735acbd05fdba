"""Seeded synthetic inputs for the MoE layer, shared by the oracle side and the
GPU side of every test and by the benchmark.

This module draws random numbers and stores them; it holds none of the
layer's arithmetic (no routing, no quantisation, no FFN).  Distributions follow
the workload definitions: x ~ N(0, 1); router and expert weights ~ N(0, 0.02^2)
(0.02 read as the standard deviation); per-expert bias ~ U(-0.1, 0.1).

Every tensor (and every expert's slice of a weight tensor) has its own stream:
a torch generator seeded from numpy's SeedSequence([seed, tensor_id, expert]).
Values depend on the device the generator runs on (torch's CPU and GPU
generators differ), so a test generates once and hands the same tensors to
both sides.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

from .configs import MoEConfig

# stream ids
X, W_GATE, BIAS, W1, W3, W2, SH_W1, SH_W3, SH_W2, TOKEN_IDS = range(10)

X_STD = 1.0
W_STD = 0.02
BIAS_HALF_WIDTH = 0.1
ZIPF_S = 1.2
ZIPF_SPAN = 2.0
VOCAB = 65536          # token-id range for the hash-router workload
TOKEN_ZIPF_S = 1.1     # token frequency ~ rank^-1.1 (text-like: few ids very common)


def _gen(device, seed: int, tensor_id: int, expert: int = 0) -> torch.Generator:
    s = np.random.SeedSequence([seed, tensor_id, expert]).generate_state(1, np.uint64)[0]
    g = torch.Generator(device=device)
    g.manual_seed(int(s) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def normal(shape, std, device, seed, tensor_id, expert=0) -> torch.Tensor:
    g = _gen(device, seed, tensor_id, expert)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def uniform(shape, lo, hi, device, seed, tensor_id) -> torch.Tensor:
    g = _gen(device, seed, tensor_id)
    t = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    return t.mul_(hi - lo).add_(lo)


def storage_dtype(cfg: MoEConfig) -> torch.dtype:
    """Element type x and the expert weights are held in before any library
    call.  fp8 workloads keep fp32 weights here: the library (and, separately,
    the oracle) quantise them to e4m3 blocks."""
    return {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float32}[cfg.dtype]


def x_dtype(cfg: MoEConfig) -> torch.dtype:
    return torch.float32 if cfg.dtype == "f32" else torch.bfloat16


def zipf_logit_offset(E: int) -> torch.Tensor:
    """Per-expert logit offset: a Zipf(s=1.2) weight over ranks 1..E (rank r =
    expert r-1), mapped affinely so rank 1 gets 2.0 and rank E gets 0.0."""
    r = np.arange(1, E + 1, dtype=np.float64)
    lo = float(E) ** (-ZIPF_S)
    off = ZIPF_SPAN * (r ** (-ZIPF_S) - lo) / (1.0 - lo)
    return torch.from_numpy(off.astype(np.float32))


def make_router(cfg: MoEConfig, device="cpu") -> Dict[str, torch.Tensor]:
    out = {
        "x": normal((cfg.T, cfg.d), X_STD, device, cfg.seed, X).to(x_dtype(cfg)),
        "w_gate": normal((cfg.d, cfg.E), W_STD, device, cfg.seed, W_GATE),
        "bias": uniform((cfg.E,), -BIAS_HALF_WIDTH, BIAS_HALF_WIDTH, device, cfg.seed, BIAS),
    }
    out["logit_offset"] = zipf_logit_offset(cfg.E).to(device) if cfg.skew else None
    return out


def expert_weights(cfg: MoEConfig, e: int, device="cpu", shared: bool = False,
                   dtype: Optional[torch.dtype] = None):
    """(w13 [2*d_ff, d], w2 [d, d_ff]) of one expert.  w13 stacks the gate
    projection W1 (rows 0..d_ff-1) over the up projection W3."""
    dt = storage_dtype(cfg) if dtype is None else dtype
    ids = (SH_W1, SH_W3, SH_W2) if shared else (W1, W3, W2)
    w1 = normal((cfg.d_ff, cfg.d), W_STD, device, cfg.seed, ids[0], e)
    w3 = normal((cfg.d_ff, cfg.d), W_STD, device, cfg.seed, ids[1], e)
    w2 = normal((cfg.d, cfg.d_ff), W_STD, device, cfg.seed, ids[2], e)
    return torch.cat([w1, w3], 0).to(dt), w2.to(dt)


def make_experts(cfg: MoEConfig, device="cpu", experts=None, dtype=None):
    """Stacked weights of the listed routed experts (default: all, or the local
    range for an expert-parallel share) and of the shared expert(s).  Filled one
    expert at a time so the full-precision temporaries stay one expert large."""
    dt = storage_dtype(cfg) if dtype is None else dtype
    if experts is None:
        experts = list(range(cfg.e_begin, cfg.e_end))
    n = len(experts)
    w13 = torch.empty((n, 2 * cfg.d_ff, cfg.d), dtype=dt, device=device)
    w2 = torch.empty((n, cfg.d, cfg.d_ff), dtype=dt, device=device)
    for i, e in enumerate(experts):
        a, b = expert_weights(cfg, e, device, dtype=dt)
        w13[i].copy_(a)
        w2[i].copy_(b)
    sh13 = torch.empty((cfg.n_shared, 2 * cfg.d_ff, cfg.d), dtype=dt, device=device)
    sh2 = torch.empty((cfg.n_shared, cfg.d, cfg.d_ff), dtype=dt, device=device)
    for i in range(cfg.n_shared):
        a, b = expert_weights(cfg, i, device, shared=True, dtype=dt)
        sh13[i].copy_(a)
        sh2[i].copy_(b)
    return {"w13": w13, "w2": w2, "sh_w13": sh13, "sh_w2": sh2, "experts": experts}


def token_ids(cfg: MoEConfig, device="cpu") -> torch.Tensor:
    """int32 [T] token ids for the hash router: ranks drawn with probability
    proportional to r^-TOKEN_ZIPF_S over r = 1..VOCAB, then mapped through a
    fixed seeded permutation of the vocabulary (so common ids are not the
    small ones)."""
    ss = np.random.SeedSequence([cfg.seed, TOKEN_IDS])
    rng = np.random.default_rng(ss)
    r = np.arange(1, VOCAB + 1, dtype=np.float64)
    p = r ** (-TOKEN_ZIPF_S)
    p /= p.sum()
    ranks = rng.choice(VOCAB, size=cfg.T, p=p)
    perm = rng.permutation(VOCAB)
    return torch.from_numpy(perm[ranks].astype(np.int32)).to(device)
