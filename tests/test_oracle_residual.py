"""Pins of the oracle's residual-channel stage ("ARCQuant" summary, gist.science,
paper 2601.07475, 'Methodology'): channels are ranked by their absolute maximum,
the top channels get a second NVFP4 stage that quantizes what the first stage
left over, and those residual blocks are appended along the reduction axis.

Each check leans on something other than the oracle's own residual code:
* the per-channel maxima and the order equal numpy's max and stable lexsort;
* the primary blocks are the row-wise quantizer's output on the gathered
  tensor (itself pinned elsewhere);
* the residual blocks are the block quantizer applied to x - v*d recomputed
  here in binary64 from the stored codes and scales (the product and the
  difference are exact in binary64, so one rounding to binary32 remains);
* a block the primary stage reconstructs exactly leaves a residual of +0
  everywhere, hence all-zero residual codes and scale;
* the two stages together reconstruct the residual channels much better than
  the primary stage alone and leave the other channels untouched.
"""
import numpy as np
import pytest

import oracle
import testkit
from oracle import AXIS_COLS, MODE_4OVER6, MODE_STD, RULE_MAE, RULE_MAX, RULE_MSE

F32 = testkit.bf16_to_f32


def unpack_codes(packed):
    p = np.asarray(packed, np.uint8).reshape(-1)
    out = np.empty(p.size * 2, np.uint8)
    out[0::2] = p & 15
    out[1::2] = p >> 4
    return out


def e2m1_values(codes):
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float64)
    v = grid[codes & 7]
    return np.where(codes & 8, -v, v)


E4M3 = np.array([oracle.e4m3_decode(s) for s in range(256)], np.float32)


def outlier_tensor(seed, rows, cols, n_out=8, factor=40.0):
    """Student-t values with a few channels scaled up, as activations with
    outlier channels look."""
    x = testkit.fill((rows, cols), testkit.STUDENT_T3, 0.5, seed)
    idx = testkit.sample(seed + 1, cols, n_out)
    testkit.scale_columns(x, idx, factor)
    return x, np.sort(idx)


def test_channel_absmax_is_column_max_of_abs():
    x = testkit.fill((37, 80), testkit.STUDENT_T3, 0.5, 11)
    x[:, 5] = 0
    x[:, 6] = 0x8000  # -0.0 everywhere
    got = oracle.channel_absmax(x)
    want = np.abs(F32(x)).max(axis=0).astype(np.float32)
    np.testing.assert_array_equal(got, want)
    assert got[5] == 0 and got[6] == 0 and not np.signbit(got[6])


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_channel_order_is_stable_descending_sort(seed):
    rng = np.random.default_rng(seed)
    a = rng.integers(0, 12, 200).astype(np.float32) * np.float32(0.25)  # many ties
    got = oracle.channel_order(a)
    want = np.lexsort((np.arange(a.size), -a.astype(np.float64)))
    np.testing.assert_array_equal(got, want)


def test_channel_order_degenerate():
    np.testing.assert_array_equal(oracle.channel_order(np.zeros(33, np.float32)), np.arange(33))
    np.testing.assert_array_equal(oracle.channel_order(np.array([2.0], np.float32)), [0])
    a = np.arange(48, dtype=np.float32)
    np.testing.assert_array_equal(oracle.channel_order(a), np.arange(47, -1, -1))


def test_outlier_channels_come_first():
    x, idx = outlier_tensor(21, 64, 256, n_out=16, factor=100.0)
    perm = oracle.channel_order(oracle.channel_absmax(x))
    assert set(perm[:16].tolist()) == set(idx.tolist())


@pytest.mark.parametrize("mode,rule", [(MODE_STD, RULE_MSE), (MODE_4OVER6, RULE_MSE),
                                       (MODE_4OVER6, RULE_MAE), (MODE_4OVER6, RULE_MAX)])
@pytest.mark.parametrize("nres", [0, 32, 256])
def test_primary_blocks_are_rowwise_quantize_of_gathered(mode, rule, nres):
    rows, cols = 12, 256
    x, _ = outlier_tensor(31, rows, cols)
    perm = oracle.channel_order(oracle.channel_absmax(x))
    r = oracle.quantize_residual(x, perm, nres, mode, rule)
    ref = oracle.quantize(np.ascontiguousarray(x[:, perm]), AXIS_COLS, mode, rule,
                          want_selmap=False, want_err=False)
    assert r["gscale"] == ref["gscale"]
    assert r["packed"].shape == (rows, (cols + nres) // 2)
    assert r["scales"].shape == (rows, (cols + nres) // 16)
    np.testing.assert_array_equal(r["packed"][:, : cols // 2].reshape(-1), ref["packed"])
    np.testing.assert_array_equal(r["scales"][:, : cols // 16].reshape(-1), ref["scales"])


@pytest.mark.parametrize("mode,rule", [(MODE_STD, RULE_MSE), (MODE_4OVER6, RULE_MSE),
                                       (MODE_4OVER6, RULE_MAE), (MODE_4OVER6, RULE_MAX)])
@pytest.mark.parametrize("nres", [16, 64, 256])
def test_residual_blocks_quantize_the_binary64_residual(mode, rule, nres):
    rows, cols = 10, 256
    x, _ = outlier_tensor(41 + nres, rows, cols)
    perm = oracle.channel_order(oracle.channel_absmax(x))
    r = oracle.quantize_residual(x, perm, nres, mode, rule)
    g = r["gscale"]
    bpr = cols // 16
    xg = F32(x[:, perm]).astype(np.float64)
    codes = unpack_codes(r["packed"]).reshape(rows, cols + nres)
    S = r["scales"]
    for row in range(rows):
        for b in range(nres // 16):
            d = np.float32(E4M3[S[row, b]] * np.float32(g))
            v = e2m1_values(codes[row, b * 16:(b + 1) * 16])
            res = (xg[row, b * 16:(b + 1) * 16] - v * np.float64(d)).astype(np.float32)
            q = oracle.quantize_block(res, g, mode, rule)
            c = q.chosen
            assert S[row, bpr + b] == q.S[c]
            want = np.array([q.code[c][i] for i in range(16)], np.uint8)
            np.testing.assert_array_equal(codes[row, cols + b * 16: cols + (b + 1) * 16], want)


def test_exact_blocks_leave_zero_residual():
    # Every block holds +-0.75 and values of the E2M1 grid times 1/8.  Under
    # 4/6 the tensor scale is 0.75 / 1536 = 2^-11, the max->6 candidate gets
    # block scale 256 and decode step 1/8, so the primary stage is exact and
    # the residual is +0 everywhere.
    rng = np.random.default_rng(5)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float32) * np.float32(0.125)
    rows, cols = 6, 128
    xf = grid[rng.integers(0, 8, (rows, cols))] * rng.choice([-1, 1], (rows, cols))
    xf[:, ::16] = np.float32(0.75) * rng.choice([-1, 1], (rows, cols // 16))
    x = (xf.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    perm = np.arange(cols, dtype=np.int32)
    for rule in (RULE_MSE, RULE_MAE, RULE_MAX):
        r = oracle.quantize_residual(x, perm, cols, MODE_4OVER6, rule)
        assert r["gscale"] == np.float32(2.0 ** -11)
        assert (r["scales"][:, : cols // 16] == 0x78).all()  # E4M3 256 = 2^8
        assert (r["packed"][:, cols // 2:] == 0).all()
        assert (r["scales"][:, cols // 16:] == 0).all()


@pytest.mark.parametrize("mode", [MODE_STD, MODE_4OVER6])
def test_two_stages_reconstruct_the_residual_channels_better(mode):
    rows, cols, nres = 32, 512, 64
    x, _ = outlier_tensor(61, rows, cols, n_out=32, factor=60.0)
    perm = oracle.channel_order(oracle.channel_absmax(x))
    r = oracle.quantize_residual(x, perm, nres, mode, RULE_MSE)
    g = r["gscale"]
    deq = oracle.dequantize(r["packed"].reshape(-1), r["scales"].reshape(-1), g, rows,
                            cols + nres, AXIS_COLS).astype(np.float64)
    prim = deq[:, :cols]
    both = prim.copy()
    both[:, :nres] += deq[:, cols:]
    xg = F32(x[:, perm]).astype(np.float64)
    e1 = np.sum((xg[:, :nres] - prim[:, :nres]) ** 2)
    e2 = np.sum((xg[:, :nres] - both[:, :nres]) ** 2)
    assert e1 > 0 and e2 < 0.05 * e1
    # Without residual channels the output is the primary stage alone.
    r0 = oracle.quantize_residual(x, perm, 0, mode, RULE_MSE, gscale=g)
    np.testing.assert_array_equal(r0["packed"], r["packed"][:, : cols // 2])


def test_given_tensor_scale_is_used():
    x, _ = outlier_tensor(71, 4, 64)
    perm = oracle.channel_order(oracle.channel_absmax(x))
    r = oracle.quantize_residual(x, perm, 16, MODE_4OVER6, RULE_MSE, gscale=np.float32(0.5))
    assert r["gscale"] == np.float32(0.5)
    ref = oracle.quantize(np.ascontiguousarray(x[:, perm]), AXIS_COLS, MODE_4OVER6, RULE_MSE,
                          gscale=np.float32(0.5), want_selmap=False, want_err=False)
    np.testing.assert_array_equal(r["scales"][:, :4].reshape(-1), ref["scales"])


@pytest.mark.parametrize("nres", [-16, 8, 80])
def test_bad_residual_count_is_rejected(nres):
    x, _ = outlier_tensor(81, 4, 64)
    with pytest.raises(ValueError):
        oracle.quantize_residual(x, np.arange(64, dtype=np.int32), nres, MODE_4OVER6, RULE_MSE)


def test_bad_permutation_entry_is_rejected():
    x, _ = outlier_tensor(82, 4, 64)
    perm = np.arange(64, dtype=np.int32)
    perm[3] = 64
    with pytest.raises(ValueError):
        oracle.quantize_residual(x, perm, 16, MODE_4OVER6, RULE_MSE)
