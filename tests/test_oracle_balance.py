"""Pins for the oracle's per-expert bias update (auxiliary-loss-free balancing)."""
import numpy as np
import pytest

from oracle import balance as B
from oracle import route as R


def _f32(v):
    return np.asarray(v, dtype=np.float32)


def test_hand_example():
    # loads 3,1,2,2: mean 2 -> the overloaded expert steps down, the underloaded one up
    out = B.bias_update([3, 1, 2, 2], _f32([0, 0, 0, 0]), 0.25)
    assert out.tolist() == [-0.25, 0.25, 0.0, 0.0]


def test_equal_loads_leave_bias_unchanged():
    bias = _f32([0.3, -0.7, 1.5, 0.0, 2.0 ** -20])
    for v in (0, 1, 7, 1000):
        assert B.bias_update([v] * 5, bias, 0.01).tolist() == bias.tolist()


def test_sign_around_a_non_integer_mean():
    # loads 1,1,2: mean 4/3, so 1 < mean < 2 (no load equals the mean)
    out = B.bias_update([1, 1, 2], _f32([0.5, -0.5, 0.1]), 0.125)
    assert out.tolist() == [0.625, -0.375, float(np.float32(np.float32(0.1) - np.float32(0.125)))]
    # mean exactly equal to some loads: those experts do not move
    out = B.bias_update([0, 3, 3, 6], _f32([1, 1, 1, 1]), 0.5)
    assert out.tolist() == [1.5, 1.0, 1.0, 0.5]


def test_addition_rounds_in_fp32():
    # 1 + 2^-30 is not an fp32 number: the step vanishes; 2^-30 + 2^-30 is exact
    g = 2.0 ** -30
    out = B.bias_update([0, 2], _f32([1.0, 2.0 ** -30]), g)
    assert out[0] == np.float32(1.0 + g) == np.float32(1.0)
    assert out[1] == np.float32(2.0 ** -30 - g) == 0.0
    out = B.bias_update([0, 2], _f32([2.0 ** -30, 1.0]), g)
    assert out[0] == np.float32(2.0 ** -29)


def test_expert_load_counts_pairs():
    idx = np.array([[0, 3], [3, 1], [2, 3]])
    assert B.expert_load(idx, 5).tolist() == [1, 1, 1, 3, 0]
    assert B.expert_load(idx, 5).sum() == idx.size


def _loop(gamma, steps, sign=1.0):
    """Route -> count -> update, repeated over fresh seeded batches on a workload
    whose logit offset favours the low-numbered experts (a dominant expert)."""
    E, G, M, k, T = 16, 4, 2, 4, 256
    gk = -(-k // M)
    rng = np.random.default_rng(7)
    offset = _f32(2.0 * (np.arange(E)[::-1] / (E - 1)) ** 3)   # expert 0 gets +2
    bias = np.zeros(E, dtype=np.float32)
    ratios = []
    for _ in range(steps):
        logits = _f32(rng.normal(size=(T, E)))
        idx, _ = R.route_from_logits(logits, bias, G, M, k, gk, offset)
        load = B.expert_load(idx, E)
        ratios.append(load.max() / load.mean())
        bias = B.bias_update(load, bias, sign * gamma)
    return ratios


def test_loop_pulls_load_off_the_dominant_expert():
    # the page's measured claim, in miniature: the update keeps the load from
    # staying on the initially dominant experts
    r = _loop(0.05, 60)
    assert r[0] > 2.5
    late = float(np.mean(r[-10:]))
    assert late < 1.6 and late < 0.6 * r[0]
    # the same loop with the step's sign flipped drives the load further onto them
    bad = _loop(0.05, 60, sign=-1.0)
    assert float(np.mean(bad[-10:])) > r[0]
    # and with no update it stays where it started
    flat = _loop(0.0, 20)
    assert abs(float(np.mean(flat)) - r[0]) < 0.5
