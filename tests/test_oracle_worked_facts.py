"""The oracle against the pages' worked facts (fixtures in tests/golden/).

Each fixture case names the page and section it restates; the expected values
in it were derived by hand from those facts, not produced by the oracle.
"""
import json
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
with open(os.path.join(HERE, "golden", "worked_facts.json")) as fh:
    CASES = json.load(fh)["cases"]

MODES = {"std": oracle.MODE_STD, "4over6": oracle.MODE_4OVER6}
RULES = {"mse": oracle.RULE_MSE, "mae": oracle.RULE_MAE}


@pytest.mark.parametrize("case", CASES, ids=[c["id"] for c in CASES])
def test_worked_fact(case):
    mode = MODES[case["mode"]]
    if "amax" in case:
        g = oracle.global_scale(case["amax"], mode)
        assert g == np.float32(case["g"])
    q = oracle.quantize_block(case["x"], case["g"], mode, RULES[case["rule"]])
    exp = case["expect"]
    assert list(q.S)[: q.ncand] == exp["S"]
    if "scale_values" in exp:
        assert [oracle.e4m3_decode(S) for S in exp["S"]] == exp["scale_values"]
    for c in range(q.ncand):
        if f"codes{c}" in exp:
            assert list(q.code[c]) == exp[f"codes{c}"]
        if f"xhat{c}" in exp:
            assert [np.float32(v) for v in q.xhat[c]] == [np.float32(v) for v in exp[f"xhat{c}"]]
        if f"err{c}" in exp:
            assert np.float32(q.err[c]) == np.float32(exp[f"err{c}"])
    if "chosen" in exp:
        assert q.chosen == exp["chosen"]


def test_two_thirds_and_full_range_under_scale6():
    """'Problem statement': with the max at 6, every value strictly between 2/3
    of the max and the max is off-grid.  Sweep bf16 values in that open range
    for a block with max 6 and g = 1: none reconstructs exactly."""
    vals = np.arange(4.0, 6.0, 2.0 ** -5, dtype=np.float32)[1:]  # all exact in bf16
    for v in vals:
        x = np.zeros(16, np.float32)
        x[0], x[1] = 6.0, v
        q = oracle.quantize_block(x, 1.0, oracle.MODE_STD, oracle.RULE_MSE)
        assert q.xhat[0][1] != v


def test_worst_error_in_the_scaled_domain_is_at_5():
    """'Problem statement': rounding near the scaled value 5 dominates the
    error; over [0, 6] the largest |E2M1(y) - y| is 1, reached at y = 5."""
    y = np.linspace(0, 6, 600001, dtype=np.float32)
    m = oracle.e2m1_index_array(y)
    grid = np.array([oracle.e2m1_decode(c) for c in range(8)], np.float32)
    err = np.abs(grid[m] - y)
    assert err.max() == 1.0
    assert np.all(y[err == 1.0] == 5.0)


def test_scale4_range_is_plus_minus_4():
    """'Core mechanism': under the max->4 candidate the block spans [-4, 4] and
    the spacing between 3 and 4 is 1."""
    rng = np.random.default_rng(2)
    for _ in range(200):
        x = rng.standard_normal(16).astype(np.float32)
        x = x * np.float32(2.0 ** rng.integers(-3, 4))
        q = oracle.quantize_block(x, 2.0 ** -3, oracle.MODE_4OVER6, oracle.RULE_MSE)
        mags = np.array(q.code[1]) & 7
        # the max element lands on 4 (index 6); rounding of the E4M3 scale can
        # push it to 3 or keep it at 4, never to 6 unless the scale saturates
        assert mags.max() <= 6


def test_dynamic_range_of_the_two_candidates():
    """'Adaptive block scaling algorithm': scaling to 4 shrinks the block's
    dynamic range; the smallest nonzero level is 1/12 of the max under scale-6
    and 1/8 under scale-4."""
    x = np.zeros(16, np.float32)
    x[0] = 12.0
    x[1] = 1.0  # exactly 1/12 of the max
    q = oracle.quantize_block(x, 0.5, oracle.MODE_4OVER6, oracle.RULE_MSE)
    # g = 0.5: S6 = 4 -> d6 = 2, y(1) = 0.5 -> code 1 (exact); S4 = 6 -> d4 = 3, 1/3 -> code 1 (1.5)
    assert q.xhat[0][1] == 1.0
    assert q.xhat[1][1] == 1.5
