"""Pins for the oracle's hash router."""
import numpy as np
import pytest

from oracle import hash_route as H
from oracle import route as R


@pytest.mark.parametrize("ctr,key", [((1, 0, 0, 0), (5, 7)), ((2, 0, 0, 0), (0, 0)),
                                     ((12345, 77, 0, 0), (2**64 - 1, 3)),
                                     ((0, 1, 0, 0), (0x0123456789ABCDEF, 0)),
                                     ((2**32 - 1, 255, 9, 2**63), (1, 2**63 + 5))])
def test_philox_matches_numpy_bit_generator(ctr, key):
    # numpy's Philox is Philox4x64-10; it increments its 256-bit counter before
    # each block, so starting it at ctr - 1 makes its first block use ctr
    c = sum(int(v) << (64 * i) for i, v in enumerate(ctr)) - 1
    start = np.array([(c >> (64 * i)) & H.MASK64 for i in range(4)], dtype=np.uint64)
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=start)
    assert [int(v) for v in bg.random_raw(4)] == H.philox4x64_10(ctr, key)


def test_experts_distinct_and_deterministic():
    ids = np.array([0, 1, 2, 2**31 - 1, 7, 1, 0, 123456, 7])
    for E, k in ((16, 4), (256, 8), (64, 6), (9, 9), (1024, 16), (5, 1)):
        idx, w = H.hash_route(ids, E, k, seed=42)
        for t in range(ids.size):
            assert len(set(idx[t].tolist())) == k
            assert idx[t].min() >= 0 and idx[t].max() < E
        # equal token ids, equal rows
        assert idx[1].tolist() == idx[5].tolist() and idx[0].tolist() == idx[6].tolist()
        assert idx[4].tolist() == idx[8].tolist()
        assert np.all(w == np.float32(1.0) / np.float32(k))
    a, _ = H.hash_route(ids, 256, 8, seed=1)
    b, _ = H.hash_route(ids, 256, 8, seed=2)
    assert not np.array_equal(a, b)              # the seed keys the hash


def test_draws_follow_the_stated_rule():
    # the first expert of a token is floor(u0 * E / 2^64) of its first Philox word
    for v in (0, 5, 99999):
        u0 = H.philox4x64_10((v, 0, 0, 0), (3, 0))[0]
        assert H.token_experts(v, 256, 4, 3)[0] == (u0 * 256) >> 64
    # negative ids are taken as their uint32 bit pattern
    assert H.token_experts(-1, 64, 4, 3) == H.token_experts(2**32 - 1, 64, 4, 3)


def test_expert_frequencies_uniform():
    E, k = 16, 4
    idx, _ = H.hash_route(np.arange(4000), E, k, seed=9)
    freq = np.bincount(idx.ravel(), minlength=E)
    exp = idx.size / E
    chi2 = float(((freq - exp) ** 2 / exp).sum())
    assert chi2 < 45.0                            # 15 dof: p ~ 1e-4


def test_fill_rule_when_draws_run_out():
    # with a budget of one block (4 draws), k = E = 8 cannot be met by draws alone:
    # the drawn experts come first, then the smallest unused ones in order
    got = H.token_experts(17, 8, 8, 5, max_blocks=1)
    drawn = []
    for u in H.philox4x64_10((17, 0, 0, 0), (5, 0)):
        e = (u * 8) >> 64
        if e not in drawn:
            drawn.append(e)
    assert got[:len(drawn)] == drawn
    assert got[len(drawn):] == [e for e in range(8) if e not in drawn]


def test_logit_weights_are_the_top_k_renormalisation():
    # when every expert is chosen (k = E, one group), the hash router's weights
    # for a token are the top-k router's weights of the same experts
    rng = np.random.default_rng(3)
    E = 8
    L = rng.normal(size=(50, E)).astype(np.float32)
    idx, w = H.hash_route(np.arange(50), E, E, seed=4, logits=L)
    ridx, rw = R.route_from_logits(L, np.zeros(E, np.float32), 1, 1, E, E)
    for t in range(50):
        # same set, so the same S up to summation order; compare per expert
        order = {int(e): j for j, e in enumerate(ridx[t])}
        s = np.array([rw[t][order[int(e)]] for e in idx[t]], dtype=np.float32)
        assert np.allclose(w[t], s, rtol=4e-7, atol=0)
        assert abs(float(w[t].astype(np.float64).sum()) - 1.0) < 4e-7
