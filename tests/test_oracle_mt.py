"""The CPU baseline's threaded driver runs the oracle's own quantizer on row
ranges after reducing the amax first; its outputs must equal the single-
threaded oracle's bit for bit (the error sum to binary64 reordering)."""
import numpy as np
import pytest

import oracle
import testkit


@pytest.mark.parametrize("rows,cols", [(1, 16), (37, 80), (64, 1024), (203, 160)])
@pytest.mark.parametrize("threads", [1, 3, 8, 64])
@pytest.mark.parametrize("mode,rule", [(oracle.MODE_STD, oracle.RULE_MSE),
                                       (oracle.MODE_4OVER6, oracle.RULE_MSE),
                                       (oracle.MODE_4OVER6, oracle.RULE_MAE),
                                       (oracle.MODE_4OVER6, oracle.RULE_MAX)])
def test_threaded_driver_equals_single_thread(rows, cols, threads, mode, rule):
    x = testkit.fill((rows, cols), testkit.STUDENT_T3, 0.5, rows * 7 + cols)
    want = oracle.quantize(x, oracle.AXIS_COLS, mode, rule)
    got = oracle.quantize_mt(x, mode, rule, threads)
    for k in ("packed", "scales", "selmap"):
        np.testing.assert_array_equal(got[k], want[k], err_msg=k)
    assert got["gscale"].view(np.uint32) == want["gscale"].view(np.uint32)
    assert abs(got["err_sum"] - want["err_sum"]) <= 1e-12 * abs(want["err_sum"])


def test_threaded_driver_with_given_scale():
    x = testkit.fill((48, 320), testkit.NORMAL, 1.0, 9)
    g = np.float32(0.013)
    want = oracle.quantize(x, oracle.AXIS_COLS, oracle.MODE_4OVER6, oracle.RULE_MSE, gscale=g)
    got = oracle.quantize_mt(x, oracle.MODE_4OVER6, oracle.RULE_MSE, 5, gscale=g)
    for k in ("packed", "scales", "selmap"):
        np.testing.assert_array_equal(got[k], want[k], err_msg=k)
    assert got["gscale"] == g
