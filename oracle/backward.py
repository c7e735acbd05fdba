"""Backward of the MoE layer forward, in fp64.

TEST INFRASTRUCTURE ONLY (see the package header).

Sources: deepmox ch.5 "The network becomes part of the forward pass" (the
backward carries its own communication and splits into the gradient for the
input and the gradient for the weights); zenaique "Why all to all dominates"
(the backward mirrors dispatch and combine with two more all-to-alls).

The pages give no formulas.  Reading: the backward is the
exact derivative of the forward the other modules define, with the expert
selection held fixed (it is piecewise constant in the logits) and no gradient
for the routing bias (it only steers selection and is moved by the balancing
rule).  Forward recap:
    L = x W_g (+ offset),  s = sqrt(softplus(L)),  w_j = s_{idx_j} / S,  S = sum_j s_{idx_j}
    xp = pack(x),  a = xp W1^T,  u = xp W3^T,  h = silu(a) u,  yp = h W2^T
    out = ysh + sum_j w_j yp[dest_j]                 (ysh: the shared expert on x)
Backward for g = d loss / d out:
    combine : d_yp[dest_j] = w_j g,   d_w_j = <g, yp[dest_j]>,   d_ysh = g
    experts : d_h = d_yp W2,  dW2 = d_yp^T h,
              da = d_h u silu'(a),  du = d_h silu(a),  silu'(a) = sig(a) (1 + a (1 - sig(a)))
              d_xp = da W1 + du W3,  dW1 = da^T xp,  dW3 = du^T xp
    dispatch: dx[t] = sum_j d_xp[dest_j]  (+ the shared expert's dx)
    gate    : ds_j = (d_w_j - sum_i w_i d_w_i) / S,
              dL[t, idx_j] = ds_j sig(L) / (2 s)   (zero for unselected experts)
              dx += dL W_g^T,  dW_g = x^T dL

Pins (tests/test_oracle_backward.py): every gradient against torch.autograd in
fp64 on the CPU (an independent implementation of the chain rule) over the same
forward with the selection fixed; finite differences on the gate path.
"""
from __future__ import annotations

import numpy as np


def _sig(z):
    return 1.0 / (1.0 + np.exp(-z))


def combine_backward(g, yp, dest, w, rows: int):
    """d_yp [rows, d] and d_w [T, k]; slots with dest = -1 get no gradient."""
    g = np.asarray(g, dtype=np.float64)
    yp = np.asarray(yp, dtype=np.float64)
    T, k = dest.shape
    d_yp = np.zeros((rows, g.shape[1]), dtype=np.float64)
    d_w = np.zeros((T, k), dtype=np.float64)
    for t in range(T):
        for j in range(k):
            r = int(dest[t, j])
            if r < 0:
                continue
            d_yp[r] = float(w[t, j]) * g[t]
            d_w[t, j] = float(np.dot(g[t], yp[r]))
    return d_yp, d_w


def expert_backward(X, w13, w2, dy):
    """One SwiGLU expert: returns (dX, dW13, dW2) in fp64."""
    X = np.asarray(X, dtype=np.float64)
    w13 = np.asarray(w13, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    d_ff = w13.shape[0] // 2
    w1, w3 = w13[:d_ff], w13[d_ff:]
    a = X @ w1.T
    u = X @ w3.T
    sg = _sig(a)
    silu = a * sg
    h = silu * u
    dh = dy @ w2
    dW2 = dy.T @ h
    da = dh * u * sg * (1.0 + a * (1.0 - sg))
    du = dh * silu
    dX = da @ w1 + du @ w3
    dW13 = np.concatenate([da.T @ X, du.T @ X], axis=0)
    return dX, dW13, dW2


def grouped_ffn_backward(xp, offsets, w13, w2, d_yp):
    """Routed experts over an expert-contiguous buffer: (d_xp, dW13 [n], dW2 [n])."""
    xp = np.asarray(xp)
    n_exp = len(offsets) - 1
    rows = int(offsets[-1])
    d = xp.shape[1]
    d_xp = np.zeros((rows, d), dtype=np.float64)
    dW13 = np.zeros((n_exp,) + np.asarray(w13[0]).shape, dtype=np.float64)
    dW2 = np.zeros((n_exp,) + np.asarray(w2[0]).shape, dtype=np.float64)
    for i in range(n_exp):
        lo, hi = int(offsets[i]), int(offsets[i + 1])
        if hi == lo:
            continue
        dX, a13, a2 = expert_backward(xp[lo:hi], w13[i], w2[i], d_yp[lo:hi])
        d_xp[lo:hi] = dX
        dW13[i] = a13
        dW2[i] = a2
    return d_xp, dW13, dW2


def dispatch_backward(d_xp, dest, T: int):
    """dx[t] = sum_j d_xp[dest[t, j]] over the slots routed to the local experts."""
    d_xp = np.asarray(d_xp, dtype=np.float64)
    dx = np.zeros((T, d_xp.shape[1]), dtype=np.float64)
    for t in range(T):
        for j in range(dest.shape[1]):
            r = int(dest[t, j])
            if r >= 0:
                dx[t] += d_xp[r]
    return dx


def gate_backward(x, w_gate, logits, idx, d_w):
    """(dx_gate [T, d], dW_g [d, E], dL [T, E]) from the gate-weight gradient.
    logits are the fp32 logits the routing used (offset included)."""
    x = np.asarray(x, dtype=np.float64)
    wg = np.asarray(w_gate, dtype=np.float64)
    L = np.asarray(logits, dtype=np.float64)
    T, E = L.shape
    k = idx.shape[1]
    dL = np.zeros((T, E), dtype=np.float64)
    for t in range(T):
        sel = [int(e) for e in idx[t]]
        lv = L[t, sel]
        s = np.sqrt(np.logaddexp(0.0, lv))
        S = s.sum()
        w = s / S
        dw = np.asarray(d_w[t], dtype=np.float64)
        ds = (dw - float(np.dot(w, dw))) / S
        for j in range(k):
            dL[t, sel[j]] = ds[j] * _sig(lv[j]) / (2.0 * s[j])
    return dL @ wg.T, x.T @ dL, dL
