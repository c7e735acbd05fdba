"""Dispatch: per-expert histogram, exclusive scan, stable permutation, pack.

Sources: deepmox ch.5 "The network becomes part of the forward pass" (a
forward chunk dispatches tokens to experts, runs the expert MLP, combines);
zenaique "Why all to all dominates MoE step time" (dispatch ships every token's
hidden state to the holders of its k experts); shivam2003 "Worked example"
(bytes = tokens x hidden x bytes x dispatch-and-return).

The packed buffer is expert-contiguous; with groups holding consecutive
experts it is also group-ordered, i.e. one GPU's all-to-all send layout.

Definition (written out as a loop, not a sort):
  counts[e]   = number of (token, slot) pairs routed to e
  offsets     = exclusive prefix sum of counts (length E+1)
  walking tokens t = 0..T-1 in order and their slots j = 0..k-1:
     r = offsets[e] + (pairs already placed for e);  dest[t,j] = r; src[r] = t
  xp[r] = x[src[r]]
An expert range [e_begin, e_end) keeps only pairs whose expert is in the range
(one expert-parallel rank's share); rows are then numbered from 0 at e_begin
and every other dest is -1.

Pins (tests/test_oracle_dispatch.py): counts sum to T*k; offsets[E] = T*k;
dest is a bijection onto [0, rows); src[dest[t,j]] = t; src increases inside
each expert segment; numpy's stable argsort of the flattened expert ids and
np.bincount give the same src and counts.
"""
from __future__ import annotations

import numpy as np


def dispatch(idx, E, e_begin=0, e_end=None):
    """Returns counts [n_local], offsets [n_local+1], dest [T,k] (-1 = not
    local), src [rows]; n_local = e_end - e_begin."""
    idx = np.asarray(idx)
    T, k = idx.shape
    if e_end is None:
        e_end = E
    n = e_end - e_begin
    counts = np.zeros(n, dtype=np.int64)
    for e in idx.ravel().tolist():
        if e_begin <= e < e_end:
            counts[e - e_begin] += 1
    offsets = np.zeros(n + 1, dtype=np.int64)
    for e in range(n):
        offsets[e + 1] = offsets[e] + counts[e]
    placed = np.zeros(n, dtype=np.int64)
    dest = np.full((T, k), -1, dtype=np.int64)
    src = np.zeros(int(offsets[n]), dtype=np.int64)
    rows = idx.tolist()
    for t in range(T):
        for j in range(k):
            e = rows[t][j]
            if not (e_begin <= e < e_end):
                continue
            le = e - e_begin
            r = int(offsets[le] + placed[le])
            placed[le] += 1
            dest[t, j] = r
            src[r] = t
    return (counts.astype(np.int32), offsets.astype(np.int32),
            dest.astype(np.int32), src.astype(np.int32))


def pack(x, src):
    """xp[r] = x[src[r]] (a plain row gather; values are copied unchanged)."""
    return np.asarray(x)[np.asarray(src, dtype=np.int64)]


def dispatch_bytes(T, k, d, in_bytes, out_bytes, scale_bytes_per_row=0):
    """Algorithmic HBM bytes of the pack: read x once, write T*k rows, read idx,
    write dest and src (4 bytes each per pair)."""
    return T * d * in_bytes + T * k * (d * out_bytes + scale_bytes_per_row) + 12 * T * k
