"""Hash router: a token's experts fixed by a hash of its token id.

TEST INFRASTRUCTURE ONLY (see the package header).

Source
  * mastering-deepseek-v4 "MoE + Expert-Parallel Overlap (Exp08)", Implemented:
    besides the affinity-based top-k router, a hash router emulates the early
    layers -- the expert set depends on the token, not on the gate.

Readings where the page is silent:
  * the hash is a published counter-based generator, Philox4x64-10 (Salmon,
    Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11),
    keyed by (seed, 0) with counter (token id as uint32, block, 0, 0); each block
    yields four 64-bit words, used in order;
  * a word u picks expert floor(u * E / 2^64); a repeat of an expert already
    chosen for the token is skipped; the k distinct experts are listed in the
    order drawn;
  * after 256 blocks (1024 draws) any slots still empty take the smallest
    unused experts in increasing order (never reached for k << E; it bounds the
    work per token);
  * no group (node) limit: the hash router does not look at groups;
  * gate weights: 1/k each, or -- when logits are given -- the unbiased
    affinities sqrt(softplus(logit)) of the chosen experts renormalised as in
    the top-k router (fp32, left-to-right sum, one division each).

Pins (tests/test_oracle_hash.py): Philox4x64-10 against numpy's Philox bit
generator (an independent implementation of the same published function);
k distinct experts per token; equal token ids get equal rows; expert frequencies
uniform within a chi-square bound; the fill rule on a forced-exhaustion case;
weights equal the top-k router's renormalisation when the hash happens to pick
the same set.
"""
from __future__ import annotations

import numpy as np

from . import affinity as _aff

f32 = np.float32
MASK64 = (1 << 64) - 1
MAX_BLOCKS = 256

# Philox4x64 multipliers and Weyl key increments (from the published definition)
_M0, _M1 = 0xD2E7470EE14C6C93, 0xCA5A826395121157
_W0, _W1 = 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B


def philox4x64_10(ctr, key):
    """One Philox4x64 block, 10 rounds.  ctr: 4 ints < 2^64, key: 2 ints < 2^64."""
    c0, c1, c2, c3 = (int(v) & MASK64 for v in ctr)
    k0, k1 = (int(v) & MASK64 for v in key)
    for _ in range(10):
        p0 = _M0 * c0
        p1 = _M1 * c2
        c0, c1, c2, c3 = ((p1 >> 64) ^ c1 ^ k0) & MASK64, p1 & MASK64, ((p0 >> 64) ^ c3 ^ k1) & MASK64, p0 & MASK64
        k0 = (k0 + _W0) & MASK64
        k1 = (k1 + _W1) & MASK64
    return [c0, c1, c2, c3]


def token_experts(token_id: int, E: int, k: int, seed: int, max_blocks: int = MAX_BLOCKS):
    """The k experts of one token, in draw order."""
    v = int(token_id) & 0xFFFFFFFF
    chosen = []
    for b in range(max_blocks):
        for u in philox4x64_10((v, b, 0, 0), (seed, 0)):
            e = (u * E) >> 64
            if e not in chosen:
                chosen.append(e)
                if len(chosen) == k:
                    return chosen
    for e in range(E):
        if len(chosen) == k:
            break
        if e not in chosen:
            chosen.append(e)
    return chosen


def hash_route(token_ids, E: int, k: int, seed: int, logits=None, max_blocks: int = MAX_BLOCKS):
    """idx [T, k] int32 and w [T, k] fp32 for token ids [T]."""
    ids = np.asarray(token_ids).reshape(-1)
    T = ids.size
    idx = np.zeros((T, k), dtype=np.int32)
    cache = {}
    for t in range(T):
        v = int(ids[t]) & 0xFFFFFFFF
        if v not in cache:
            cache[v] = token_experts(v, E, k, seed, max_blocks)
        idx[t] = cache[v]
    if logits is None:
        w = np.full((T, k), f32(1.0) / f32(k), dtype=np.float32)
        return idx, w
    L = np.asarray(logits, dtype=np.float32)
    s = _aff.affinity(np.take_along_axis(L, idx.astype(np.int64), axis=1))
    S = s[:, 0].copy()
    for j in range(1, k):
        S = (S + s[:, j]).astype(np.float32)
    w = (s / S[:, None]).astype(np.float32)
    return idx, w
