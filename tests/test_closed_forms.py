"""Closed forms the pages state for one token-expert pair."""
import json
import os

from moe_inputs import configs as C
from oracle import combine as Cb, dispatch as D

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_crossover_printed_value():
    g = json.load(open(os.path.join(GOLD, "crossover.json")))
    cfg = C.FLASH.with_(d=g["d"], d_ff=g["d_ff"])
    flops = C.flops_per_pair(cfg)
    # fp8 dispatch row + bf16 combine row, per pair
    byts = (D.dispatch_bytes(1, 1, cfg.d, 0, 1) - 12) + (Cb.combine_bytes(1, 1, cfg.d, 2, 0, shared=False) - 8)
    assert flops == g["flops_per_pair"]
    assert byts == g["bytes_per_pair"] == 3 * cfg.d
    assert flops // byts == g["crossover_flops_per_byte"] == 2 * cfg.d_ff


def test_v3_gemm_flops():
    cfg = C.V3
    total = (cfg.pairs + cfg.T) * C.flops_per_pair(cfg)
    assert total == 12_987_981_103_104
