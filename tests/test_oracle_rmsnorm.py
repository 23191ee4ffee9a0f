"""Pins of the oracle's RMSNorm, the normalisation the outlier-channel path can
apply before its two quantization stages ("ARCQuant" summary, gist.science
2601.07475, 'Methodology': the authors' fused kernel covers channel
reordering, RMSNorm and both stages).

The page names RMSNorm but not its arithmetic; the oracle fixes a summation
order (8-element partial sums, then a pairwise tree) and uses IEEE sqrt and
division.  These checks lean on what holds whatever the order:
* rstd against the binary64 value 1/sqrt(mean(x^2) + eps), within the error
  the few binary32 roundings allow;
* y within one bf16 step of x * rstd computed in binary64;
* constant rows normalise to exactly +-1; with eps = 0, scaling a row by a
  power of two leaves y unchanged bit for bit;
* a weight of 1 changes nothing, a weight of 2 doubles y exactly, and a
  weight multiplies after the first rounding to bf16.
"""
import numpy as np
import pytest

import oracle
import testkit

F32 = testkit.bf16_to_f32


def to_bf16(f):
    """Round binary32 values to bf16 bit patterns (nearest even)."""
    u = np.asarray(f, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("cols", [8, 64, 80, 1040, 5120])
@pytest.mark.parametrize("eps", [0.0, 1e-6, 1e-2])
def test_rstd_matches_binary64(cols, eps):
    x = testkit.fill((6, cols), testkit.STUDENT_T3, 0.5, 7 + cols)
    xf = F32(x).astype(np.float64)
    for r in range(x.shape[0]):
        want = 1.0 / np.sqrt(np.mean(xf[r] ** 2) + np.float64(np.float32(eps)))
        got = np.float64(oracle.rms_rstd(x[r], eps))
        assert abs(got - want) <= 4e-6 * want, (r, got, want)


@pytest.mark.parametrize("cols", [64, 5120])
def test_y_within_one_bf16_step_of_binary64(cols):
    x = testkit.fill((8, cols), testkit.NORMAL, 3.0, 11)
    eps = 1e-5
    y = F32(oracle.rmsnorm(x, None, eps)).astype(np.float64)
    xf = F32(x).astype(np.float64)
    rstd = 1.0 / np.sqrt(np.mean(xf ** 2, axis=1, keepdims=True) + np.float64(np.float32(eps)))
    exact = xf * rstd
    step = np.abs(exact) * 2.0 ** -7  # one bf16 step at that magnitude (8 significant bits)
    assert np.all(np.abs(y - exact) <= step + 1e-30)


@pytest.mark.parametrize("c", [1.5, -0.25, 3.0])
def test_constant_rows_normalise_to_one(c):
    cols = 128
    x = np.full((3, cols), to_bf16(np.float32(c)), np.uint16)
    y = F32(oracle.rmsnorm(x, None, 0.0))
    np.testing.assert_array_equal(y, np.full_like(y, np.sign(c)))


@pytest.mark.parametrize("k", [-20, -3, 5, 30])
def test_power_of_two_scaling_leaves_y_unchanged(k):
    x = testkit.fill((5, 256), testkit.STUDENT_T3, 0.5, 21)
    xs = to_bf16(F32(x) * np.float32(2.0 ** k))
    np.testing.assert_array_equal(F32(xs), F32(x) * np.float32(2.0 ** k))  # exact scaling
    np.testing.assert_array_equal(oracle.rmsnorm(xs, None, 0.0), oracle.rmsnorm(x, None, 0.0))


def test_weight_steps():
    x = testkit.fill((4, 96), testkit.NORMAL, 1.0, 31)
    eps = 1e-6
    y = oracle.rmsnorm(x, None, eps)
    ones = np.full(96, to_bf16(np.float32(1.0)), np.uint16)
    twos = np.full(96, to_bf16(np.float32(2.0)), np.uint16)
    np.testing.assert_array_equal(oracle.rmsnorm(x, ones, eps), y)
    np.testing.assert_array_equal(F32(oracle.rmsnorm(x, twos, eps)), 2.0 * F32(y))
    w = testkit.fill((96,), testkit.NORMAL, 1.0, 32)
    yw = oracle.rmsnorm(x, w, eps)
    np.testing.assert_array_equal(yw, to_bf16(F32(w)[None, :] * F32(y)))


def test_zero_row_with_eps_and_bad_shapes():
    x = np.zeros((2, 64), np.uint16)
    y = oracle.rmsnorm(x, None, 1e-6)
    assert (y == 0).all()
    with pytest.raises(ValueError):
        oracle.rmsnorm(np.zeros((2, 12), np.uint16), None, 1e-6)
