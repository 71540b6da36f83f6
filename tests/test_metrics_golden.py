"""The performance-model arithmetic against the values the pages print
(tests/golden/pages_worked_values.json; each entry cites its page and section)."""
import json
import os

import pytest

from tiled_software_pipelined_amd import metrics

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_worked_values.json")))


@pytest.mark.parametrize("row", GOLDEN["timings_4096"]["rows"], ids=[r[0] for r in GOLDEN["timings_4096"]["rows"]])
def test_tflops_matches_printed_timings(row):
    g = GOLDEN["timings_4096"]
    _, ms, tf = row
    assert abs(metrics.tflops(g["M"], g["N"], g["K"], ms * 1e-3) - tf) <= g["tolerance_tflops"]


def test_flops_is_2mnk():
    assert metrics.flops(4096, 4096, 4096) == 137438953472
    assert metrics.flops(4095, 4097, 4104) == 2 * 4095 * 4097 * 4104


def test_stage_budget_table():
    g = GOLDEN["stage_budget"]
    per = metrics.stage_bytes(g["BM"], g["BN"], g["BK"], g["esize"])
    assert per == g["per_stage_kib"] * 1024
    assert g["BM"] * g["BK"] * g["esize"] == g["a_tile_kib"] * 1024
    assert g["BK"] * g["BN"] * g["esize"] == g["b_tile_kib"] * 1024
    for s, kib in g["stages_kib"].items():
        assert int(s) * per == kib * 1024


def test_naive_intensity():
    g = GOLDEN["naive_intensity"]
    for K in (1, 256, 4096):
        assert metrics.naive_intensity(K, g["esize"]) == g["value"]


def test_block_tile_intensity():
    g = GOLDEN["block_tile_intensity"]
    assert metrics.tile_intensity(g["BM"], g["BN"], g["BK"], g["esize"]) == g["value"]
    # independent of BK, and largest at BM = BN for a fixed BM + BN (section 4.3)
    assert metrics.tile_intensity(128, 128, 32, 4) == g["value"]
    assert metrics.tile_intensity(64, 192, 8, 4) < g["value"]


def test_balance_point():
    g = GOLDEN["balance_v100"]
    assert abs(metrics.balance_point(g["peak_flops"], g["bandwidth"]) - g["value"]) <= g["tolerance"]


def test_bk8_tile_bytes():
    g = GOLDEN["bk8_tile_bytes"]
    assert g["BM"] * g["BK"] * g["esize"] == g["kib"] * 1024


def test_roofline_time_picks_the_binding_limit():
    # bf16 4096^3: compute-bound at 2.5 PF / 8 TB/s; 4096^2 x 256: memory-bound
    t = metrics.roofline_time(4096, 4096, 4096, 2, 4, 2.5e15, 8e12)
    assert t == pytest.approx(137438953472 / 2.5e15)
    t = metrics.roofline_time(4096, 4096, 256, 2, 4, 2.5e15, 8e12)
    assert t == pytest.approx(metrics.algorithmic_bytes(4096, 4096, 256, 2, 4) / 8e12)
