"""Router: gate logits, biased node-limited top-k selection, gate weights.

Sources
  * mastering-deepseek-v4 "MoE + Expert-Parallel Overlap (Exp08)", Implemented:
    top-k gating over Sqrt(Softplus(.)) affinities; balancing by a per-expert
    bias (no auxiliary loss).
  * zenaique "MoE node-limited routing" (opening definition; Real products:
    M=4 over 256 experts): a token's experts live on at most M nodes.
  * deepnotes "DeepSeek-V3 671B: the real parallelism mesh", The real cluster:
    4 consecutive experts per GPU, so a node holds a contiguous expert range.

Readings where the pages are silent:
  * group g holds experts [g*E/G, (g+1)*E/G)  (consecutive placement);
  * a group's score is the sum of its gk = ceil(k/M) largest biased
    affinities, added in descending order in fp32;
  * the M highest-scoring groups are kept, ties to the lower group index;
  * experts outside the kept groups are excluded (not scored 0);
  * the k chosen experts are the highest biased affinities among the kept
    groups, ties to the lower expert index, listed in that order;
  * gate weights come from the unbiased affinities: w_j = s_j / S with
    S the fp32 left-to-right sum of s over the chosen list; no extra scale.

Logits (O1) are formed in fp64 from the exact inputs and rounded to fp32;
everything after them is fp32 with one rounding per operation, so the GPU,
given the same fp32 logits, must reproduce indices and weights bit for bit.
"""
from __future__ import annotations

import numpy as np

from . import affinity as _aff

f32 = np.float32


def gate_logits(x, w_gate):
    """L = x @ W_g, computed in fp64 from the exact fp32/bf16-valued inputs,
    rounded once to fp32.  x [T, d], w_gate [d, E]."""
    x64 = np.asarray(x, dtype=np.float64)
    w64 = np.asarray(w_gate, dtype=np.float64)
    return (x64 @ w64).astype(np.float32)


def scores(logits, bias, logit_offset=None):
    """s = sqrt(softplus(l)), b = s + bias; l = logits (+ offset, fp32 add)."""
    l = np.asarray(logits, dtype=np.float32)
    if logit_offset is not None:
        l = l + np.asarray(logit_offset, dtype=np.float32)
    s = _aff.affinity(l)
    b = s + np.asarray(bias, dtype=np.float32)
    return s, b


def group_scores(b, G, gk):
    """[T, G]: per group, its gk largest biased affinities summed largest first."""
    T, E = b.shape
    bg = np.asarray(b, dtype=np.float32).reshape(T, G, E // G)
    top = -np.sort(-bg, axis=2)[:, :, :gk]          # descending
    acc = top[:, :, 0].copy()
    for i in range(1, gk):
        acc = acc + top[:, :, i]
    return acc.astype(np.float32)


def _order_desc(v):
    """Indices sorting each row by value descending, equal values by index
    ascending (a stable sort of the negated values)."""
    return np.argsort(-v, axis=-1, kind="stable")


def select(s, b, G, M, k, gk):
    """Node-limited top-k.  Returns idx [T,k] int32 (desc. biased score),
    w [T,k] fp32, kept-group mask [T,G] bool."""
    s = np.asarray(s, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    T, E = b.shape
    gsz = E // G
    gs = group_scores(b, G, gk)
    kept_groups = _order_desc(gs)[:, :M]
    gmask = np.zeros((T, G), dtype=bool)
    np.put_along_axis(gmask, kept_groups, True, axis=1)
    emask = np.repeat(gmask, gsz, axis=1)
    masked = np.where(emask, b, -np.inf).astype(np.float32)
    idx = _order_desc(masked)[:, :k].astype(np.int32)
    sel = np.take_along_axis(s, idx, axis=1)
    S = sel[:, 0].copy()
    for j in range(1, k):
        S = S + sel[:, j]
    w = (sel / S[:, None]).astype(np.float32)
    return idx, w, gmask


def route_from_logits(logits, bias, G, M, k, gk, logit_offset=None):
    s, b = scores(logits, bias, logit_offset)
    idx, w, gmask = select(s, b, G, M, k, gk)
    return idx, w


def route(x, w_gate, bias, G, M, k, gk, logit_offset=None):
    L = gate_logits(x, w_gate)
    idx, w = route_from_logits(L, bias, G, M, k, gk, logit_offset)
    return L, idx, w
