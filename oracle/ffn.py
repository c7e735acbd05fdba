"""Expert FFN: SwiGLU routed experts and the shared expert, in fp64.

Sources: mastering-deepseek-v4 "MoE + Expert-Parallel Overlap (Exp08)",
Implemented: shared experts are always active, routed experts are
fine-grained; each token-expert pair costs 6*d*d_ff flops (three d x d_ff
matrices).  The pages do not spell out the expert MLP; the reading used here
is SwiGLU (Shazeer 2020, "GLU Variants Improve Transformer") without biases:

    a = x W1^T,  u = x W3^T,  h = a * sigmoid(a) * u,  y = h W2^T

with weights stored [out, in]: w13 = [W1; W3] is [2*d_ff, d] and w2 is
[d, d_ff].  h is kept in full precision here (the GPU rounds it to its
storage type between the two products).

Pins (tests/test_oracle_ffn.py): a hand-derived worked example
(tests/golden/swiglu_worked.json) for expert_forward and for expert_hidden
(h = 1.5 ln3 there; a W1/W3 swap gives 2 sigmoid(2) ln3); expert_hidden
followed by h W2^T equals expert_forward; flop counter equal to 6*d*d_ff per
row; the dense evaluation (every expert on every token, gated by a T x E
matrix) equals dispatch -> ffn -> combine.
"""
from __future__ import annotations

import numpy as np


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def expert_forward(X, w13, w2):
    """One SwiGLU expert on rows X [n, d] -> [n, d], fp64.  Returns (y, flops)."""
    X = np.asarray(X, dtype=np.float64)
    w13 = np.asarray(w13, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    d_ff = w13.shape[0] // 2
    w1, w3 = w13[:d_ff], w13[d_ff:]
    a = X @ w1.T
    u = X @ w3.T
    h = a * sigmoid(a) * u
    y = h @ w2.T
    n, d = X.shape
    flops = 2 * n * (2 * d_ff) * d + 2 * n * d * d_ff
    return y, flops


def expert_hidden(X, w13):
    """h = silu(X W1^T) * (X W3^T) in fp64 (used by the fp8 emulation)."""
    X = np.asarray(X, dtype=np.float64)
    w13 = np.asarray(w13, dtype=np.float64)
    d_ff = w13.shape[0] // 2
    a = X @ w13[:d_ff].T
    u = X @ w13[d_ff:].T
    return a * sigmoid(a) * u


def grouped_ffn(xp, offsets, w13, w2, weight_fn=None):
    """Routed experts over an expert-contiguous buffer: rows
    [offsets[i], offsets[i+1]) of xp go through expert i.  w13/w2 are stacked
    per local expert, or weight_fn(i) -> (w13_i, w2_i) supplies them one at a
    time.  Returns (yp [rows, d] fp64, flops)."""
    xp = np.asarray(xp)
    n_exp = len(offsets) - 1
    rows = int(offsets[-1])
    d = xp.shape[1] if xp.ndim == 2 else None
    yp = np.zeros((rows, d), dtype=np.float64)
    flops = 0
    for i in range(n_exp):
        lo, hi = int(offsets[i]), int(offsets[i + 1])
        if hi == lo:
            continue
        a, b = weight_fn(i) if weight_fn is not None else (w13[i], w2[i])
        y, f = expert_forward(xp[lo:hi], a, b)
        yp[lo:hi] = y
        flops += f
    return yp, flops
