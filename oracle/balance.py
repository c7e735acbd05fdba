"""Auxiliary-loss-free load balancing: the per-expert bias update.

TEST INFRASTRUCTURE ONLY (see the package header).

Source
  * mastering-deepseek-v4 "MoE + Expert-Parallel Overlap (Exp08)", Implemented:
    expert load is balanced by updating a per-expert bias rather than by an
    auxiliary loss; Measured: the bias keeps the load from collapsing onto the
    expert that dominates at the start.

Reading where the page is silent: after a batch, each
expert's bias moves one fixed step gamma towards balance,

    bias_e <- bias_e + gamma * sign(mean_load - load_e),

where load_e counts the (token, slot) pairs routed to e in the batch,
mean_load = sum(load) / E and sign(0) = 0.  The comparison is exact (rational
arithmetic); the update is one fp32 addition of +gamma or -gamma, or nothing.
The bias only shifts which experts are selected; the gate weights keep using
the unbiased affinities (the route module).

Pins (tests/test_oracle_balance.py): a hand-computed example; equal loads leave
the bias unchanged; the sign at an exactly representable tie and around a
non-integer mean; the fp32 rounding of the addition; and the loop that the page
measures -- route, count, update, repeated on a skewed workload -- lowering the
max/mean load, which a flipped sign or a dropped update would not do.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

f32 = np.float32


def expert_load(idx, E: int) -> np.ndarray:
    """Pairs routed to each expert: load[e] = #{(t, j) : idx[t, j] == e}."""
    flat = np.asarray(idx).reshape(-1)
    load = np.zeros(E, dtype=np.int64)
    for e in flat:
        load[int(e)] += 1
    return load


def bias_update(load, bias, gamma: float) -> np.ndarray:
    """One update step; returns the new fp32 bias (the input is not modified)."""
    load = [int(v) for v in np.asarray(load).reshape(-1)]
    E = len(load)
    mean = Fraction(sum(load), E)
    out = np.array(bias, dtype=np.float32).copy()
    g = f32(gamma)
    for e in range(E):
        diff = mean - load[e]
        s = (diff > 0) - (diff < 0)
        if s > 0:
            out[e] = f32(out[e] + g)
        elif s < 0:
            out[e] = f32(out[e] - g)
    return out
