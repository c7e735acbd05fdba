"""Pins for the oracle's affinity s = sqrt(softplus(l)) (fp32 from fp32 logits).

Pinned against fp64 libm (np.logaddexp, np.sqrt) and against values fixed by
mathematics: the exact function is strictly increasing, so the fp32 result
must be non-decreasing over every fp32 logit, and it must be the correctly
rounded value wherever fp64 libm can tell which that is.  Both are checked
exhaustively over every fp32 logit in [-210, 88] (about 2.25e9 values, split
over the host's cores); below -210 and above 88 the closed forms in
test_special_values apply.
"""
import concurrent.futures as cf
import os

import numpy as np

from oracle import affinity as A

LO = np.float32(-210.0)
HI = np.float32(88.0)
CHUNK = 1 << 22


def _ascending(b0, n, negative):
    """n consecutive fp32 values in ascending order starting at bit pattern
    b0 (for negatives the bit patterns run downwards)."""
    if negative:
        return (np.uint32(b0) - np.arange(n, dtype=np.uint32)).view(np.float32)
    return (np.uint32(b0) + np.arange(n, dtype=np.uint32)).view(np.float32)


def _check_range(args):
    """Checks one run of consecutive logits.  Returns (first s, last s, order
    violations, disagreements with fp64 libm, of which near a rounding
    boundary)."""
    b0, n, negative = args
    l = _ascending(b0, n, negative)
    s = A.affinity(l)
    viol = int(np.count_nonzero(s[1:] < s[:-1]))
    ref64 = np.sqrt(np.logaddexp(0.0, l.astype(np.float64)))
    ref32 = ref64.astype(np.float32)
    bad = np.nonzero(s != ref32)[0]
    near = 0
    if bad.size:
        r64, r32 = ref64[bad], ref32[bad]
        other = np.nextafter(r32, np.where(r64 > r32.astype(np.float64), np.float32(np.inf), np.float32(0)))
        mid = (r32.astype(np.float64) + other.astype(np.float64)) * 0.5
        close = np.abs(r64 - mid) <= 2.0 ** -44 * r64
        near = int(np.count_nonzero(close & (s[bad] == other)))
    return float(s[0]), float(s[-1]), viol, int(bad.size), near


def _runs():
    """The fp32 logits in [LO, HI] in ascending order, as runs of CHUNK."""
    runs = []
    top = int(LO.view(np.uint32))          # bits of -210; -0.0 is 0x80000000
    b = top
    while b >= 0x80000000:
        n = min(CHUNK, b - 0x80000000 + 1)
        runs.append((b, n, True))
        b -= n
    end = int(HI.view(np.uint32))
    b = 1                                   # +0.0 equals -0.0: start after it
    while b <= end:
        n = min(CHUNK, end - b + 1)
        runs.append((b, n, False))
        b += n
    return runs


def test_exhaustive_monotone_and_correctly_rounded():
    runs = _runs()
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with cf.ProcessPoolExecutor(workers) as ex:
        res = list(ex.map(_check_range, runs, chunksize=4))
    viol = sum(r[2] for r in res)
    # across run boundaries
    viol += sum(1 for a, b in zip(res, res[1:]) if b[0] < a[1])
    bad = sum(r[3] for r in res)
    near = sum(r[4] for r in res)
    n = sum(r[1] for r in runs)
    print(f"{n} logits: {viol} order violations, {bad} differ from fp64 libm, {near} of them "
          f"within 2^-44 of a rounding boundary")
    assert n > 2_200_000_000
    assert viol == 0
    # every disagreement is one where the fp64 reference itself cannot decide
    # the rounding, and our value is the other neighbour
    assert bad == near
    assert bad <= 64


def test_special_values():
    assert A.affinity(np.float32(0.0)) == np.float32(np.sqrt(np.log(2.0)))
    assert A.affinity(np.float32(-0.0)) == A.affinity(np.float32(0.0))
    # once e^-l is below half an fp64 ulp of l, softplus(l) = l and s = fp32(sqrt(l))
    for l in [np.float32(40.0), np.float32(87.5), np.float32(300.5), np.float32(1e6), np.float32(3.4e38)]:
        assert float(A.softplus64(np.float32(l))) == float(l)
        assert A.affinity(l) == np.float32(np.sqrt(np.float64(l)))
    # large negative logits: s = e^{l/2} to fp32, and 0 once that is below
    # half the smallest fp32 subnormal (l < -2*103.97)
    for l in [-30.0, -87.0, -150.0, -200.0]:
        assert A.affinity(np.float32(l)) == np.float32(np.exp(l / 2.0))
    assert A.affinity(np.float32(-210.0)) == 0.0
    assert A.affinity(np.float32(-1e30)) == 0.0


def test_branch_edges_continuous():
    # the Taylor branch (|l| < 2^-14) and the general form meet without a step:
    # both sides of each edge agree with fp64 libm
    for edge in (2.0 ** -14, -(2.0 ** -14)):
        b = np.float32(edge).view(np.uint32)
        l = (b + np.arange(-2000, 2000).astype(np.int64)).astype(np.uint32).view(np.float32)
        l = np.sort(l)
        s = A.affinity(l)
        assert np.all(np.diff(s.astype(np.float64)) >= 0)
        ref = np.sqrt(np.logaddexp(0.0, l.astype(np.float64))).astype(np.float32)
        assert np.array_equal(s, ref)


def test_exp_neg_and_log1p_pieces():
    a = np.linspace(0, 300, 400001)
    e = A.exp_neg(a)
    ref = np.exp(-a)
    assert np.max(np.abs(e - ref) / ref) <= 4 * 2.0 ** -53
    u = np.linspace(0, 1, 400001)
    g = A.log1p_unit(u)
    ref = np.log1p(u)
    ok = u > 0
    assert np.max(np.abs(g[ok] - ref[ok]) / ref[ok]) <= 8 * 2.0 ** -53
    assert A.log1p_unit(np.float64(0.0)) == 0.0
    tiny = np.float64(1e-300)
    assert A.log1p_unit(tiny) == tiny
