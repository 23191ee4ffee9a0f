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


# ---------------------------------------------------------------------------
# Order-independent pin.  Rows of small dyadic values (at most 4 significant
# bits, exponents in a narrow window) have squares that are integer multiples
# of one unit, and every partial sum of them stays below 2^24 units, so every
# summation order gives the same, exact binary32 sum of squares.  rstd and y
# then follow from the RMSNorm definition alone, each step one correctly
# rounded binary32 operation (numpy float32 division and sqrt are IEEE), and
# the oracle must match bit for bit whatever order it sums in.


def _exact_rows(rows, cols, seed, max_k):
    """bf16 rows of k * 2^e (|k| <= max_k, e in {-3, -2, -1}) whose squares
    sum exactly in binary32 under any order; returns (bits, exact_ss)."""
    rng = np.random.default_rng(seed)
    k = rng.integers(-max_k, max_k + 1, size=(rows, cols))
    e = rng.integers(-3, 0, size=(rows, cols))
    units = (k.astype(np.int64) ** 2) << (2 * (e + 3))  # x^2 in units of 2^-6
    total = units.sum(axis=1)
    assert total.max() < 2 ** 24, "every partial sum must be exact in binary32"
    xf = (k * np.ldexp(1.0, e)).astype(np.float32)
    bits = xf.view(np.uint32) >> 16
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), xf)  # exact bf16
    return bits.astype(np.uint16), total.astype(np.float64) * 2.0 ** -6


@pytest.mark.parametrize("cols,max_k", [(16, 15), (64, 15), (80, 15), (1040, 15), (5120, 15),
                                        (8192, 11)])
@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.25])
def test_rstd_and_y_exact_when_the_sum_is_order_free(cols, max_k, eps):
    x, ss = _exact_rows(5, cols, 100 + cols, max_k)
    f32 = np.float32
    for r in range(x.shape[0]):
        if ss[r] == 0 and eps == 0:
            continue  # 1/sqrt(0) is outside the contract of a normalisation
        ms = f32(ss[r]) / f32(cols)          # ss is exact in binary32
        want = f32(1.0) / np.sqrt(ms + f32(eps))
        got = np.float32(oracle.rms_rstd(x[r], eps))
        assert got.view(np.uint32) == want.view(np.uint32), (r, got, want)
    keep = ~((ss == 0) & (eps == 0))
    y = oracle.rmsnorm(x[keep], None, eps)
    rstd = np.array([f32(1.0) / np.sqrt(f32(s) / f32(cols) + f32(eps)) for s in ss[keep]],
                    np.float32)
    np.testing.assert_array_equal(y, to_bf16(F32(x[keep]) * rstd[:, None]))
    w = testkit.fill((cols,), testkit.NORMAL, 1.0, 5 + cols)
    np.testing.assert_array_equal(oracle.rmsnorm(x[keep], w, eps),
                                  to_bf16(F32(w)[None, :] * F32(y)))


# ---------------------------------------------------------------------------
# The stated order on sums that do round.  This restates the order the
# oracle's header fixes (8-element fma chunks, zero padding to a power of two
# of at least 64 entries, pairwise levels) in numpy binary32 and checks that
# the oracle follows it, on rows chosen so that a plain left-to-right sum and
# the pairwise sum differ: a mistake in the tree (a dropped or misplaced
# level, a chunk of the wrong width, no padding) changes the result here.
# It checks the oracle against its own stated reading, which the page does
# not fix.


def _stated_order_ss(row_f32):
    n = row_f32.size // 8
    chunks = np.zeros(n, np.float32)
    for v in range(n):
        t = np.float32(0.0)
        for i in range(8):
            xv = row_f32[8 * v + i]
            t = np.float32(np.float64(xv) * np.float64(xv) + np.float64(t))  # one rounding (fma)
        chunks[v] = t
    p = 64
    while p < n:
        p *= 2
    a = np.zeros(p, np.float32)
    a[:n] = chunks
    while a.size > 1:
        a = (a[0::2] + a[1::2]).astype(np.float32)
    return a[0]


@pytest.mark.parametrize("cols", [8, 64, 520, 1024, 5120])
def test_rstd_follows_the_stated_pairwise_order(cols):
    x = testkit.fill((8, cols), testkit.STUDENT_T3, 0.5, 300 + cols)
    xf = F32(x)
    differs = 0
    for r in range(x.shape[0]):
        ss = _stated_order_ss(xf[r])
        seq = np.float32(0.0)
        for v in xf[r]:
            seq = np.float32(np.float64(v) * np.float64(v) + np.float64(seq))
        differs += int(seq != ss)
        want = np.float32(1.0) / np.sqrt(ss / np.float32(cols) + np.float32(1e-6))
        got = np.float32(oracle.rms_rstd(x[r], 1e-6))
        assert got.view(np.uint32) == want.view(np.uint32), (r, got, want)
    if cols >= 520:
        assert differs > 0, "inputs must separate sequential from pairwise order"
