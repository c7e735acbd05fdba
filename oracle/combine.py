"""Combine: gate-weighted sum of the expert outputs back in token order.

Sources: deepmox ch.5 "The network becomes part of the forward pass" (the
forward chunk ends by combining the expert outputs); zenaique "Why all to all
dominates MoE step time" (combine ships FFN outputs back to the token's GPU).

    out[t] = ysh[t] + sum_j w[t,j] * yp[dest[t,j]]     (slots with dest = -1,
                                                        i.e. not local, skipped)

Accumulated in fp64.  With ``out_init`` the sum is added onto an existing
buffer (one expert-parallel rank scatter-adding its share); there is then no
shared-expert term.

Pins (tests/test_oracle_combine.py): identity experts give (sum_j w)*x; a
one-hot gate reduces the combine to a gather; the dense evaluation in
test_oracle_ffn agrees.
"""
from __future__ import annotations

import numpy as np


def combine(yp, dest, w, ysh=None, out_init=None):
    dest = np.asarray(dest)
    w = np.asarray(w, dtype=np.float64)
    yp = np.asarray(yp, dtype=np.float64)
    T, k = dest.shape
    d = yp.shape[1]
    if out_init is not None:
        out = np.array(out_init, dtype=np.float64, copy=True)
    elif ysh is not None:
        out = np.array(ysh, dtype=np.float64, copy=True)
    else:
        out = np.zeros((T, d), dtype=np.float64)
    for j in range(k):
        r = dest[:, j]
        ok = r >= 0
        out[ok] += w[ok, j, None] * yp[r[ok]]
    return out


def combine_bytes(T, k, d, y_bytes, out_bytes, shared=True, accumulate=False):
    """Algorithmic HBM bytes: read k expert rows per token, dest and w
    (4+4 bytes per pair), the shared row, and write (or read+write) out."""
    b = T * k * (d * y_bytes + 8)
    if shared:
        b += T * d * y_bytes
    b += T * d * out_bytes * (2 if accumulate else 1)
    return b
