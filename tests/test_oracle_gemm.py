"""Pins of the oracle's W4A4 product: out[m][n] = ga * gb * sum_k a(m,k) b(n,k)
for two NVFP4 tensors blocked along the reduction axis, with a = v * dec(S)
(W4A4 linear layers: "Why Gated DeltaNet ... withstands 4-bit quantization",
'Background'; the augmented product over K_in + S: "ARCQuant" summary,
'Methodology').

Each check leans on something other than the oracle's own product code:
* exact rational sums (Python Fractions) with scales decoded by torch's
  float8_e4m3fn on tiny inputs;
* numpy's integer matmul when every scale is 1 and g = 1;
* a one-hot activation picks one weight element (closed form);
* concatenation along K adds the two products (the augmented identity);
* numpy's binary64 matmul of the pinned dequantizer's output, within the
  dequantizer's two roundings;
* the weight side of the augmented product repeats the primary blocks, and
  the augmented product is closer to the bf16 product X W^T than the plain
  W4A4 product on activations with outlier channels.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import testkit
from oracle import AXIS_COLS, MODE_4OVER6, MODE_STD, RULE_MSE

GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
        Fraction(4), Fraction(6)]


def random_nvfp4(rng, rows, K, scale_lo=0x00, scale_hi=0x7E):
    """Random codes and E4M3 scale bytes (NaN byte 0x7F excluded)."""
    packed = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    scales = rng.integers(scale_lo, scale_hi + 1, (rows, K // 16), dtype=np.uint8)
    return packed, scales


def torch_e4m3(S):
    return torch.from_numpy(np.ascontiguousarray(S, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def exact_values(packed, scales):
    """Element values v * dec(S) as Fractions (dec from torch's float8_e4m3fn)."""
    rows, half = packed.shape
    K = half * 2
    dec = torch_e4m3(scales)
    out = []
    for r in range(rows):
        row = []
        for k in range(K):
            byte = int(packed[r, k // 2])
            code = byte >> 4 if k & 1 else byte & 15
            v = GRID[code & 7] * (-1 if code & 8 else 1)
            row.append(v * Fraction(float(dec[r, k // 16])))
        out.append(row)
    return out


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_tiny_products_match_exact_rationals(seed):
    rng = np.random.default_rng(seed)
    M, N, K = 3, 4, 48
    pa, sa = random_nvfp4(rng, M, K)
    pb, sb = random_nvfp4(rng, N, K)
    ga, gb = np.float32(rng.uniform(1e-3, 2.0)), np.float32(rng.uniform(1e-3, 2.0))
    got, gabs = oracle.gemm(pa, sa, ga, pb, sb, gb, M, N, K, want_abs=True)
    A, B = exact_values(pa, sa), exact_values(pb, sb)
    g = Fraction(float(ga)) * Fraction(float(gb))
    for m in range(M):
        for n in range(N):
            s = sum(A[m][k] * B[n][k] for k in range(K))
            a = sum(abs(A[m][k] * B[n][k]) for k in range(K))
            want, want_abs = float(g * s), float(g * a)
            assert abs(got[m, n] - want) <= 2 * K * 2.0 ** -53 * want_abs, (m, n)
            assert abs(gabs[m, n] - want_abs) <= 2 * K * 2.0 ** -53 * want_abs, (m, n)


def test_unit_scales_match_integer_matmul():
    rng = np.random.default_rng(7)
    M, N, K = 17, 23, 320
    pa, _ = random_nvfp4(rng, M, K)
    pb, _ = random_nvfp4(rng, N, K)
    one = np.full((M, K // 16), 0x38, np.uint8)  # E4M3 1.0
    oneb = np.full((N, K // 16), 0x38, np.uint8)
    got = oracle.gemm(pa, one, 1.0, pb, oneb, 1.0, M, N, K)

    def twice_v(packed):  # 2v as integers, read straight from the nibbles
        codes = np.empty((packed.shape[0], packed.shape[1] * 2), np.int64)
        codes[:, 0::2] = packed & 15
        codes[:, 1::2] = packed >> 4
        mag = np.array([0, 1, 2, 3, 4, 6, 8, 12], np.int64)[codes & 7]
        return np.where(codes & 8, -mag, mag)

    want = twice_v(pa) @ twice_v(pb).T  # = 4 * sum v_a v_b, exact
    np.testing.assert_array_equal(got * 4, want.astype(np.float64))


def test_one_hot_activation_selects_a_weight_element():
    rng = np.random.default_rng(11)
    N, K = 9, 64
    pb, sb = random_nvfp4(rng, N, K)
    ks = [0, 1, 17, 63]
    M = len(ks)
    pa = np.zeros((M, K // 2), np.uint8)
    sa = np.full((M, K // 16), 0x38, np.uint8)
    for m, k in enumerate(ks):
        pa[m, k // 2] = 2 << (4 * (k & 1))  # code 2 = +1.0 at position k
    gb = np.float32(0.25)
    got = oracle.gemm(pa, sa, 1.0, pb, sb, gb, M, N, K)
    B = exact_values(pb, sb)
    for m, k in enumerate(ks):
        for n in range(N):
            assert got[m, n] == float(B[n][k]) * 0.25


def test_concatenation_along_k_adds_the_products():
    rng = np.random.default_rng(13)
    M, N, K1, K2 = 6, 5, 96, 32
    pa1, sa1 = random_nvfp4(rng, M, K1, 0x20, 0x50)
    pa2, sa2 = random_nvfp4(rng, M, K2, 0x20, 0x50)
    pb1, sb1 = random_nvfp4(rng, N, K1, 0x20, 0x50)
    pb2, sb2 = random_nvfp4(rng, N, K2, 0x20, 0x50)
    cat = lambda a, b: np.concatenate([a, b], axis=1)
    whole, wabs = oracle.gemm(cat(pa1, pa2), cat(sa1, sa2), 0.5, cat(pb1, pb2), cat(sb1, sb2),
                              0.75, M, N, K1 + K2, want_abs=True)
    parts = (oracle.gemm(pa1, sa1, 0.5, pb1, sb1, 0.75, M, N, K1) +
             oracle.gemm(pa2, sa2, 0.5, pb2, sb2, 0.75, M, N, K2))
    assert np.all(np.abs(whole - parts) <= 4 * (K1 + K2) * 2.0 ** -53 * wabs)


@pytest.mark.parametrize("mode", [MODE_STD, MODE_4OVER6])
def test_round_trip_matches_dequantized_matmul(mode):
    M, N, K = 40, 24, 256
    x = testkit.fill((M, K), testkit.STUDENT_T3, 0.5, 17)
    w = testkit.fill((N, K), testkit.NORMAL, 0.02, 18)
    qx = oracle.quantize(x, AXIS_COLS, mode, RULE_MSE, want_selmap=False, want_err=False)
    qw = oracle.quantize(w, AXIS_COLS, mode, RULE_MSE, want_selmap=False, want_err=False)
    got, gabs = oracle.gemm(qx["packed"], qx["scales"], qx["gscale"], qw["packed"], qw["scales"],
                            qw["gscale"], M, N, K, want_abs=True)
    dx = oracle.dequantize(qx["packed"], qx["scales"], qx["gscale"], M, K, AXIS_COLS)
    dw = oracle.dequantize(qw["packed"], qw["scales"], qw["gscale"], N, K, AXIS_COLS)
    want = dx.astype(np.float64) @ dw.astype(np.float64).T
    # Each dequantized value is v*dec(S)*g up to two binary32 roundings.
    assert np.all(np.abs(got - want) <= 2.0 ** -21 * gabs + 1e-300)


def test_duplicate_mode_repeats_the_primary_blocks():
    rows, cols, nres = 12, 128, 32
    w = testkit.fill((rows, cols), testkit.NORMAL, 0.02, 23)
    perm = np.random.default_rng(3).permutation(cols).astype(np.int32)
    q = oracle.quantize_residual(w, perm, nres, MODE_4OVER6, RULE_MSE, duplicate=True)
    ref = oracle.quantize(np.ascontiguousarray(w[:, perm]), AXIS_COLS, MODE_4OVER6, RULE_MSE,
                          want_selmap=False, want_err=False)
    assert q["gscale"] == ref["gscale"]
    np.testing.assert_array_equal(q["packed"][:, : cols // 2].reshape(-1), ref["packed"])
    np.testing.assert_array_equal(q["scales"][:, : cols // 16].reshape(-1), ref["scales"])
    np.testing.assert_array_equal(q["packed"][:, cols // 2:], q["packed"][:, : nres // 2])
    np.testing.assert_array_equal(q["scales"][:, cols // 16:], q["scales"][:, : nres // 16])


@pytest.mark.parametrize("mode", [MODE_STD, MODE_4OVER6])
def test_augmented_product_is_closer_to_the_bf16_product(mode):
    M, N, K, S = 64, 48, 512, 64
    x = testkit.fill((M, K), testkit.STUDENT_T3, 0.5, 29)
    idx = testkit.sample(30, K, 16)
    testkit.scale_columns(x, idx, 60.0)
    w = testkit.fill((N, K), testkit.NORMAL, 0.02, 31)
    exact = testkit.bf16_to_f32(x).astype(np.float64) @ testkit.bf16_to_f32(w).astype(np.float64).T
    perm = oracle.channel_order(oracle.channel_absmax(x))
    qa = oracle.quantize_residual(x, perm, S, mode, RULE_MSE)
    qb = oracle.quantize_residual(w, perm, S, mode, RULE_MSE, duplicate=True)
    aug = oracle.gemm(qa["packed"], qa["scales"], qa["gscale"], qb["packed"], qb["scales"],
                      qb["gscale"], M, N, K + S)
    pa = oracle.quantize_residual(x, perm, 0, mode, RULE_MSE)
    pb = oracle.quantize_residual(w, perm, 0, mode, RULE_MSE)
    plain = oracle.gemm(pa["packed"], pa["scales"], pa["gscale"], pb["packed"], pb["scales"],
                        pb["gscale"], M, N, K)
    e_aug = np.sum((aug - exact) ** 2)
    e_plain = np.sum((plain - exact) ** 2)
    assert e_aug < 0.8 * e_plain, (e_aug, e_plain)


def test_bad_shapes_are_rejected():
    z = np.zeros(8, np.uint8)
    with pytest.raises(ValueError):
        oracle.gemm(z, z[:1], 1.0, z, z[:1], 1.0, 1, 1, 8)  # K not a multiple of 16
    with pytest.raises(ValueError):
        oracle.gemm(z, z[:1], 1.0, z, z[:1], 1.0, 1, 1, 32)  # sizes do not match K
