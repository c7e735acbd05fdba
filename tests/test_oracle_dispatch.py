"""Pins for the oracle's dispatch (histogram, scan, stable permutation, pack)."""
import numpy as np
import pytest

from oracle import dispatch as D


def _random_idx(rng, T, E, k):
    return np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("T,E,k", [(256, 16, 4), (1000, 64, 6), (300, 256, 8), (1, 8, 3), (0, 8, 2)])
def test_invariants_and_library_pin(T, E, k):
    rng = np.random.default_rng(T + E + k)
    idx = _random_idx(rng, T, E, k) if T else np.zeros((0, k), np.int32)
    counts, offsets, dest, src = D.dispatch(idx, E)
    assert counts.sum() == T * k and offsets[-1] == T * k and offsets[0] == 0
    assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    # dest is a bijection onto [0, T*k) and src inverts it
    assert np.array_equal(np.sort(dest.ravel()), np.arange(T * k))
    tt = np.repeat(np.arange(T), k).reshape(T, k)
    assert np.array_equal(src[dest], tt)
    # the stable sort of the flattened expert ids gives the same row order
    order = np.argsort(idx.ravel(), kind="stable")
    assert np.array_equal(src, order // k)
    # rows of expert e sit in [offsets[e], offsets[e+1]), tokens increasing
    for e in range(E):
        seg = src[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert all(e in idx[t] for t in seg.tolist())


def test_group_order_is_expert_order():
    # with consecutive experts per group, the expert-contiguous buffer is also
    # group-contiguous: group g's rows are [offsets[g*E/G], offsets[(g+1)*E/G])
    rng = np.random.default_rng(5)
    T, E, G, k = 500, 32, 4, 4
    idx = _random_idx(rng, T, E, k)
    _, offsets, _, src = D.dispatch(idx, E)
    gsz = E // G
    for g in range(G):
        lo, hi = offsets[g * gsz], offsets[(g + 1) * gsz]
        seg = np.arange(lo, hi)
        # each row in the group segment belongs to an expert of that group
        e_of_row = np.repeat(np.arange(E), np.diff(offsets))
        assert np.all(e_of_row[seg] // gsz == g)


def test_expert_range():
    rng = np.random.default_rng(9)
    T, E, k = 400, 32, 4
    idx = _random_idx(rng, T, E, k)
    full_c, full_o, full_d, full_s = D.dispatch(idx, E)
    eb, ee = 4, 8
    c, o, d, s = D.dispatch(idx, E, eb, ee)
    assert np.array_equal(c, full_c[eb:ee])
    assert np.array_equal(o, full_o[eb:ee + 1] - full_o[eb])
    local = (idx >= eb) & (idx < ee)
    assert np.all(d[~local] == -1)
    assert np.array_equal(d[local], full_d[local] - full_o[eb])
    assert np.array_equal(s, full_s[full_o[eb]:full_o[ee]])


def test_pack_copies_rows():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((50, 8)).astype(np.float32)
    idx = _random_idx(rng, 50, 10, 3)
    _, _, dest, src = D.dispatch(idx, 10)
    xp = D.pack(x, src)
    for t in range(50):
        for j in range(3):
            assert np.array_equal(xp[dest[t, j]], x[t])


def test_bytes_closed_form():
    # fp8 dispatch (1 B) + bf16 combine (2 B) = 3*d bytes per token-expert pair
    d = 7168
    per_pair_dispatch = D.dispatch_bytes(1, 1, d, 0, 1) - 12
    assert per_pair_dispatch == d
