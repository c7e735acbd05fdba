"""Pins for the exposed/hidden communication model (moe_expert_routing_sqrt_amd.overlap):
the page's printed crossover, its measured saturation at 2x and the linear
growth of exposed communication below the crossover, plus limits that any
steady-state overlap model must satisfy."""
import json
import math
import os

import pytest

from moe_expert_routing_sqrt_amd import overlap as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_crossover_is_the_printed_value():
    g = json.load(open(os.path.join(GOLD, "crossover.json")))
    vc, vm = O.pair_volumes(g["d"], g["d_ff"])
    assert vc == g["flops_per_pair"] and vm == g["bytes_per_pair"]
    assert O.crossover_intensity(g["d"], g["d_ff"]) == g["crossover_flops_per_byte"]
    # independent of d: the crossover is 2 * d_ff
    assert O.crossover_intensity(7168, 2048) == 4096


def test_speedup_saturates_at_two_at_the_crossover():
    C, d, d_ff = 1.0e15, 7168, 2048
    Bx = O.crossover_bandwidth(C, d, d_ff)
    at = O.model(C, Bx, d, d_ff)
    assert at["speedup"] == pytest.approx(2.0, rel=1e-12)
    assert at["comm_to_comp"] == pytest.approx(1.0, rel=1e-12)   # the one-to-one point
    assert at["exposed"] == pytest.approx(0.0, abs=1e-24)
    for f in (0.01, 0.3, 0.9, 1.1, 3.0, 100.0):
        r = O.model(C, f * Bx, d, d_ff)
        assert 1.0 < r["speedup"] < 2.0
    assert O.model(C, 1e-6 * Bx, d, d_ff)["speedup"] == pytest.approx(1.0, rel=1e-5)
    assert O.model(C, 1e6 * Bx, d, d_ff)["speedup"] == pytest.approx(1.0, rel=1e-5)


def test_exposed_communication_linear_below_the_crossover():
    C, d, d_ff = 8.0e14, 2048, 2048
    Bx = O.crossover_bandwidth(C, d, d_ff)
    pts = [(1.0 / B, O.model(C, B, d, d_ff, pairs=1000)["exposed"]) for B in (0.2 * Bx, 0.4 * Bx, 0.8 * Bx)]
    (x0, y0), (x1, y1), (x2, y2) = pts
    assert (y1 - y0) * (x2 - x0) == pytest.approx((y2 - y0) * (x1 - x0), rel=1e-12)
    # slope = V_comm per pair times pairs; intercept = -t_comp
    slope = (y1 - y0) / (x1 - x0)
    assert slope == pytest.approx(1000 * 3 * d, rel=1e-12)
    # above the crossover nothing is exposed and utilization is 1
    above = O.model(C, 1.5 * Bx, d, d_ff, pairs=1000)
    assert above["exposed"] == 0.0 and above["utilization"] == 1.0


def test_utilization_and_time_identities():
    C, d, d_ff = 9.5e14, 7168, 2048
    Bx = O.crossover_bandwidth(C, d, d_ff)
    for f in (0.05, 0.5, 1.0, 2.0):
        r = O.model(C, f * Bx, d, d_ff, pairs=131072)
        assert r["utilization"] == pytest.approx(min(1.0, f), rel=1e-12)
        assert r["hidden"] + r["exposed"] == pytest.approx(r["t_comm"], rel=1e-12)
        assert r["serial"] == pytest.approx(r["t_comp"] + r["t_comm"], rel=1e-12)
        assert r["overlapped"] == pytest.approx(r["t_comp"] + r["exposed"], rel=1e-12)


def test_xgmi_mesh_bandwidth():
    assert math.isinf(O.ep_bandwidth(1))
    assert O.ep_bandwidth(8) == pytest.approx(8 * 153e9)
    assert O.ep_bandwidth(2) == pytest.approx(2 * 153e9)
    with pytest.raises(ValueError):
        O.ep_bandwidth(9)
