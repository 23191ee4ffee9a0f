"""Tensor-level pins of the oracle: layout, invariants, metamorphic relations,
brute force on tiny inputs and degenerate cases.

None of these re-types the oracle's block pipeline; each checks a property
that the method or the mathematics fixes:
* every reconstructed element is the nearest of the 16 E2M1 codes times the
  block's decode scale (brute force over all codes, in binary64);
* the kept candidate has the smaller error, recomputed in binary64 from the
  stored codes and scales ("Technical summary: Four Over Six (4/6)",
  'Adaptive block scaling algorithm');
* the per-tensor error statistic equals the binary64 sum of squared (or
  absolute) reconstruction errors;
* scaling by powers of two, negation, row permutation and transposition act
  on the outputs as they must.
"""
import numpy as np
import pytest
import torch

import oracle
import testkit
from oracle import AXIS_COLS, AXIS_ROWS, MODE_4OVER6, MODE_STD, RULE_MAE, RULE_MAX, RULE_MSE

F32 = testkit.bf16_to_f32


def unpack_codes(packed):
    p = np.asarray(packed, np.uint8)
    out = np.empty(p.size * 2, np.uint8)
    out[0::2] = p & 15
    out[1::2] = p >> 4
    return out


def e2m1_values(codes):
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float64)
    v = grid[codes & 7]
    return np.where(codes & 8, -v, v)


def e4m3_values(S):
    return np.array([oracle.e4m3_decode(int(s)) for s in range(256)], np.float64)[S]


def small(seed, rows=8, cols=64, scale=1.0, dist=testkit.NORMAL):
    return testkit.fill((rows, cols), dist, scale, seed)


# ------------------------------------------------------------ layout ----

@pytest.mark.parametrize("mode,rule", [(MODE_STD, RULE_MSE), (MODE_4OVER6, RULE_MSE),
                                       (MODE_4OVER6, RULE_MAE)])
def test_tensor_outputs_are_the_blocks_outputs(mode, rule):
    x = small(101, 6, 96, dist=testkit.STUDENT_T3)
    r = oracle.quantize(x, AXIS_COLS, mode, rule)
    g = r["gscale"]
    assert g == np.float32(np.float32(np.abs(F32(x)).max()) / np.float32(1536 if mode else 2688))
    codes = unpack_codes(r["packed"])
    xf = F32(x).reshape(-1, 16)
    total = 0.0
    for blk in range(xf.shape[0]):
        q = oracle.quantize_block(xf[blk], g, mode, rule)
        c = q.chosen
        assert list(codes[blk * 16:(blk + 1) * 16]) == list(q.code[c])  # even element = low nibble
        assert r["scales"][blk] == q.S[c]
        assert ((r["selmap"][blk >> 3] >> (blk & 7)) & 1) == c  # LSB-first, 1 = max->4
        total += float(np.float32(q.err[c]))
    assert r["err_sum"] == total


def test_dequantize_reproduces_reconstruction_bitwise():
    x = small(202, 4, 128, scale=3.0)
    r = oracle.quantize(x, AXIS_COLS, MODE_4OVER6, RULE_MSE)
    out = oracle.dequantize(r["packed"], r["scales"], r["gscale"], 4, 128, AXIS_COLS)
    xf = F32(x).reshape(-1, 16)
    for blk in range(xf.shape[0]):
        q = oracle.quantize_block(xf[blk], r["gscale"], MODE_4OVER6, RULE_MSE)
        np.testing.assert_array_equal(out.reshape(-1, 16)[blk].view(np.uint32),
                                      np.array(q.xhat[q.chosen], np.float32).view(np.uint32))
    out16 = oracle.dequantize(r["packed"], r["scales"], r["gscale"], 4, 128, AXIS_COLS, True)
    want16 = torch.from_numpy(out).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(out16, want16)


# ------------------------------------------------------------ brute force ----

@pytest.mark.parametrize("seed", range(6))
def test_every_element_is_nearest_code_brute_force(seed):
    rng = np.random.default_rng(seed)
    all_codes = np.arange(16, dtype=np.uint8)
    for _ in range(60):
        x = (rng.standard_normal(16) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32)
        x = F32(torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
        g = np.float32(np.abs(x).max() * rng.uniform(0.5, 2.0) / 1536)
        q = oracle.quantize_block(x, g, MODE_4OVER6, RULE_MSE)
        for c in range(2):
            d = float(q.d[c])
            cand = e2m1_values(all_codes) * d  # binary64 reconstructions of all 16 codes
            for i in range(16):
                best = np.min(np.abs(cand - float(x[i])))
                mine = abs(float(q.xhat[c][i]) - float(x[i]))
                # nearest up to the rounding of the scaled value (a few ulps)
                assert mine <= best + 4e-7 * (abs(float(x[i])) + d * 6), (seed, c, i)


@pytest.mark.parametrize("rule", [RULE_MSE, RULE_MAE])
def test_kept_candidate_has_smaller_error_binary64(rule):
    rng = np.random.default_rng(31 + rule)
    decided = 0
    for _ in range(400):
        x = (rng.standard_t(3, size=16) * 0.5).astype(np.float32)
        x = F32(torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
        g = np.float32(np.abs(x).max() * rng.uniform(0.9, 3.0) / 1536)
        q = oracle.quantize_block(x, g, MODE_4OVER6, rule)
        errs = []
        for c in range(2):
            xhat = e2m1_values(np.array(q.code[c])) * float(e4m3_values(q.S[c])) * float(g)
            dlt = xhat - x.astype(np.float64)
            errs.append(np.sum(dlt * dlt) if rule == RULE_MSE else np.sum(np.abs(dlt)))
        if abs(errs[0] - errs[1]) > 1e-5 * max(errs):
            decided += 1
            assert q.chosen == int(errs[1] < errs[0])
        else:
            assert q.chosen in (0, 1)
    assert decided > 300


def test_max_rule_error_is_largest_single_rounding_difference():
    """Minimum-maximum-error rule ("Technical summary: Four Over Six (4/6)",
    "Adaptive block scaling algorithm"): each candidate's error is the largest
    |v*d - x| over the block.  v*d - x is exact in binary64 (v has 2
    significant bits, d 24, x 8), so its single rounding to binary32 is
    np.float32 of the binary64 value; the maximum is exact."""
    rng = np.random.default_rng(41)
    decided = 0
    for _ in range(400):
        x = (rng.standard_t(3, size=16) * 0.5).astype(np.float32)
        x = F32(torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
        g = np.float32(np.abs(x).max() * rng.uniform(0.9, 3.0) / 1536)
        q = oracle.quantize_block(x, g, MODE_4OVER6, RULE_MAX)
        errs = []
        for c in range(2):
            d = float(np.float32(float(e4m3_values(q.S[c])) * float(g)))  # d = RN(dec(S) * g)
            assert np.float32(d) == np.float32(q.d[c])
            dlt = e2m1_values(np.array(q.code[c])) * d - x.astype(np.float64)
            errs.append(np.max(np.abs(dlt.astype(np.float32))))
            assert np.float32(q.err[c]) == errs[-1]
        assert q.chosen == int(errs[1] < errs[0])  # exact: ties keep max->6
        decided += errs[0] != errs[1]
    assert decided > 300


def test_max_rule_bounds_and_invariances():
    """max |delta| lies between sqrt(SSE/16) and sqrt(SSE) of the same
    candidate, scales exactly with powers of two and ignores the sign."""
    x = small(77, 4, 64, dist=testkit.STUDENT_T3).reshape(-1, 16)
    for blk in x:
        xf = F32(blk)
        g = np.float32(np.abs(xf).max() / 1536)
        qm = oracle.quantize_block(xf, g, MODE_4OVER6, RULE_MAX)
        qs = oracle.quantize_block(xf, g, MODE_4OVER6, RULE_MSE)
        for c in range(2):
            assert list(qm.code[c]) == list(qs.code[c])  # the rule changes only the choice
            sse = float(np.sum(np.square(np.array(qs.delta[c], np.float64))))
            assert np.sqrt(sse / 16) * (1 - 1e-6) <= qm.err[c] <= np.sqrt(sse) * (1 + 1e-6)
        q2 = oracle.quantize_block(xf * np.float32(4), g * np.float32(4), MODE_4OVER6, RULE_MAX)
        qn = oracle.quantize_block(-xf, g, MODE_4OVER6, RULE_MAX)
        for c in range(2):
            assert q2.err[c] == np.float32(4) * qm.err[c]
            assert qn.err[c] == qm.err[c]
        assert q2.chosen == qm.chosen == qn.chosen


def test_max_rule_on_the_three_quarters_block():
    """The block of the 'Core mechanism' worked fact ([4, 3, -3, 0, ...],
    g = 1): max->6 reconstructs 4.125, 2.75, -2.75 (largest error 0.25),
    max->4 reconstructs exactly, so the max rule keeps max->4 as well."""
    x = np.zeros(16, np.float32)
    x[:3] = [4.0, 3.0, -3.0]
    q = oracle.quantize_block(x, 1.0, MODE_4OVER6, RULE_MAX)
    assert q.err[0] == np.float32(0.25) and q.err[1] == 0.0 and q.chosen == 1


def test_tie_goes_to_scale6():
    x = np.zeros(16, np.float32)  # both candidates have zero error
    q = oracle.quantize_block(x, 1.0, MODE_4OVER6, RULE_MSE)
    assert q.err[0] == q.err[1] == 0 and q.chosen == 0
    x[0] = 6.0  # exact on both candidates: scales 1.0 and 1.5 (g = 1), codes 6 and 4
    q = oracle.quantize_block(x, 1.0, MODE_4OVER6, RULE_MSE)
    assert list(q.S) == [0x38, 0x3C]
    assert q.err[0] == q.err[1] == 0 and q.chosen == 0


# ------------------------------------------------------------ statistics ----

@pytest.mark.parametrize("mode,rule", [(MODE_STD, RULE_MSE), (MODE_4OVER6, RULE_MSE),
                                       (MODE_4OVER6, RULE_MAE), (MODE_4OVER6, RULE_MAX)])
def test_err_sum_equals_binary64_recompute(mode, rule):
    x = small(303, 32, 512, dist=testkit.STUDENT_T3)
    r = oracle.quantize(x, AXIS_COLS, mode, rule)
    xhat = oracle.dequantize(r["packed"], r["scales"], r["gscale"], 32, 512, AXIS_COLS)
    dlt = xhat.astype(np.float64) - F32(x).astype(np.float64)
    if mode == MODE_4OVER6 and rule == RULE_MAE:
        want = np.sum(np.abs(dlt))
    elif mode == MODE_4OVER6 and rule == RULE_MAX:  # sum over blocks of the block maximum
        want = np.sum(np.max(np.abs(dlt).reshape(-1, 16), axis=1))
    else:
        want = np.sum(dlt * dlt)
    assert r["err_sum"] == pytest.approx(want, rel=1e-6)


def test_four_over_six_lowers_error_on_outlier_activations():
    """The method's claim ('Technical summary: Four Over Six (4/6)', 'Key
    contributions'): choosing between the two scales brings the quantized
    tensor closer to the original than standard NVFP4."""
    x = testkit.make(2, rows=256)
    e_std = oracle.quantize(x, AXIS_COLS, MODE_STD, RULE_MSE)["err_sum"]
    e_46 = oracle.quantize(x, AXIS_COLS, MODE_4OVER6, RULE_MSE)["err_sum"]
    assert e_46 < 0.9 * e_std


def test_scale_bytes_stay_in_range():
    x = testkit.make(4, rows=64)
    r46 = oracle.quantize(x, AXIS_COLS, MODE_4OVER6, RULE_MSE)
    rst = oracle.quantize(x, AXIS_COLS, MODE_STD, RULE_MSE)
    assert r46["scales"].max() <= 0x7C  # 384 = 1.5 * 256
    assert rst["scales"].max() == 0x7E  # the amax block reaches 448
    # scale-4 is 1.5x scale-6 before E4M3 rounding
    xf = F32(x).reshape(-1, 16)
    for blk in range(0, xf.shape[0], 97):
        q = oracle.quantize_block(xf[blk], r46["gscale"], MODE_4OVER6, RULE_MSE)
        s6, s4 = float(q.s[0]), float(q.s[1])
        assert abs(4 * s4 - 6 * s6) <= 4 * np.spacing(np.float32(max(s4, 1e-30))) * 6


# ------------------------------------------------------------ metamorphic ----

def test_power_of_two_scaling_is_transparent():
    x = small(404, 8, 64, scale=0.37)
    base = oracle.quantize(x, AXIS_COLS, MODE_4OVER6, RULE_MSE)
    for k in (-20, -3, 5, 30):
        xs = torch.from_numpy(F32(x) * np.float32(2.0 ** k)).to(torch.bfloat16)
        xs = xs.view(torch.int16).numpy().view(np.uint16)
        r = oracle.quantize(xs, AXIS_COLS, MODE_4OVER6, RULE_MSE)
        np.testing.assert_array_equal(r["packed"], base["packed"])
        np.testing.assert_array_equal(r["scales"], base["scales"])
        np.testing.assert_array_equal(r["selmap"], base["selmap"])
        assert r["gscale"] == np.float32(base["gscale"] * np.float32(2.0 ** k))


def test_negation_flips_sign_bits_only():
    x = small(505, 8, 64)
    neg = x ^ np.uint16(0x8000)
    a = oracle.quantize(x, AXIS_COLS, MODE_4OVER6, RULE_MAE)
    b = oracle.quantize(neg, AXIS_COLS, MODE_4OVER6, RULE_MAE)
    np.testing.assert_array_equal(b["packed"], a["packed"] ^ np.uint8(0x88))
    np.testing.assert_array_equal(b["scales"], a["scales"])
    np.testing.assert_array_equal(b["selmap"], a["selmap"])
    assert a["err_sum"] == b["err_sum"]


def test_row_permutation_permutes_outputs():
    x = small(606, 16, 32)
    perm = np.random.default_rng(0).permutation(16)
    a = oracle.quantize(x, AXIS_COLS, MODE_4OVER6, RULE_MSE)
    b = oracle.quantize(x[perm], AXIS_COLS, MODE_4OVER6, RULE_MSE)
    np.testing.assert_array_equal(b["packed"].reshape(16, -1), a["packed"].reshape(16, -1)[perm])
    np.testing.assert_array_equal(b["scales"].reshape(16, -1), a["scales"].reshape(16, -1)[perm])


def test_column_blocks_are_row_blocks_of_the_transpose():
    x = small(707, 48, 40, scale=1e-3)
    a = oracle.quantize(x, AXIS_ROWS, MODE_4OVER6, RULE_MAE)
    b = oracle.quantize(np.ascontiguousarray(x.T), AXIS_COLS, MODE_4OVER6, RULE_MAE)
    for key in ("packed", "scales", "selmap"):
        np.testing.assert_array_equal(a[key], b[key])
    assert a["gscale"] == b["gscale"] and a["err_sum"] == b["err_sum"]
    da = oracle.dequantize(a["packed"], a["scales"], a["gscale"], 48, 40, AXIS_ROWS)
    db = oracle.dequantize(b["packed"], b["scales"], b["gscale"], 40, 48, AXIS_COLS)
    np.testing.assert_array_equal(da, db.T)


# ------------------------------------------------------------ degenerate ----

def test_all_zero_tensor_and_signed_zero():
    x = np.zeros((2, 32), np.uint16)
    x[1, 3] = 0x8000  # -0
    r = oracle.quantize(x, AXIS_COLS, MODE_4OVER6, RULE_MSE)
    assert r["gscale"] == 0 and r["err_sum"] == 0
    assert (r["scales"] == 0).all()
    codes = unpack_codes(r["packed"])
    assert codes[32 + 3] == 8 and codes.sum() == 8  # the sign of -0 is kept


def test_subnormal_and_zero_block_scales():
    # g = 1: a block max of 0.02 gives s6 = 0.00333 (E4M3 subnormal), and a
    # block max of 0.001 gives s <= 2^-10 -> scale 0 -> all codes 0.
    x = np.zeros(16, np.float32)
    x[:3] = [0.02, -0.01, 0.005]
    q = oracle.quantize_block(x, 1.0, MODE_4OVER6, RULE_MSE)
    assert 0 < q.S[0] < 8 and 0 < q.S[1] < 8
    x = np.zeros(16, np.float32)
    x[:2] = [0.001, -0.0005]
    q = oracle.quantize_block(x, 1.0, MODE_4OVER6, RULE_MSE)
    assert q.S[0] == 0 and q.S[1] == 0
    assert list(q.code[0][:2]) == [0, 8] and q.xhat[0][0] == 0
    # a zero scale reconstructs zeros, so the block error is the sum of squares
    want = float(np.float32(0.001)) ** 2 + float(np.float32(0.0005)) ** 2
    assert float(q.err[0]) == pytest.approx(want, rel=2 ** -22)


def test_given_scale_too_small_saturates():
    x = np.zeros(16, np.float32)
    x[:2] = [100.0, 30.0]
    q = oracle.quantize_block(x, 1e-3, MODE_4OVER6, RULE_MSE)  # s would be ~1.7e4
    assert q.S[0] == 0x7E and q.S[1] == 0x7E
    assert q.code[0][0] == 7  # y = 100 / 0.448 >> 6 saturates to 6


@pytest.mark.parametrize("g", [0.0, 1e-40, np.float32(2.0 ** -129)])
def test_degenerate_global_scale_encodes_zero(g):
    x = np.zeros(16, np.float32)
    x[:2] = [1e-39, -3e-40]
    q = oracle.quantize_block(x, g, MODE_4OVER6, RULE_MSE)
    assert q.S[0] == q.S[1] == 0
    assert all(c & 7 == 0 for c in q.code[0])


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros((2, 24), np.uint16), AXIS_COLS, MODE_STD, RULE_MSE)
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros((24, 16), np.uint16), AXIS_ROWS, MODE_STD, RULE_MSE)
