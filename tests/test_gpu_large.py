"""Tensors past the library's per-launch segment limits, checked on sampled
rows or columns against the oracle (the oracle on the whole 2^30-element
tensor would take a minute; the rows sampled include every segment seam).

One 65600 x 16384 bf16 tensor (2^30 + 2^20 elements, 2 GiB) covers:
  * the row quantizer's split at 2^26 blocks (block 2^26 starts row 65536),
  * the dequantizer's splits at 2^25 and 2^26 blocks,
  * the amax pass's split at 2^27 16-byte vectors (element 2^30),
and a 16384 x 65600 view of the same bytes exercises the column-blocked
kernel's 64-bit addressing on a tensor larger than 2^31 bytes.  A 140000 x
8192 tensor (2.3 GB) does the same for the outlier-channel calls, and a
1.1M-row activation operand (2.25 GB of codes) for the W4A4 product.
"""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_wave64_amd as nv
import oracle
import testkit

pytestmark = pytest.mark.gpu

ROWS, COLS = 65600, 16384
SEAM_ROWS = [0, 1, 32767, 32768, 65535, 65536, 65537, ROWS - 1]  # 2^25 / 2^26 block seams


def banner(msg):
    print(f"\n[gpu-large] {msg}", flush=True)


@pytest.fixture(scope="module")
def big():
    banner(f"generating {ROWS}x{COLS}")
    x = testkit.fill((ROWS, COLS), testkit.STUDENT_T3, 0.5, 0x5E6)
    xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    g_ref = oracle.global_scale(oracle.amax(x), nv.MODE_4OVER6)
    yield x, xd, g_ref
    del xd
    torch.cuda.empty_cache()


def sample_rows():
    rng = np.random.default_rng(3)
    return np.unique(np.concatenate([SEAM_ROWS, rng.integers(0, ROWS, 24)]))


def test_large_amax_and_global_scale(big):
    x, xd, g_ref = big
    banner("amax over 2^30 + 2^20 elements")
    a = nv.amax(xd.view(-1))
    assert a.cpu().numpy()[0].view(np.uint32) == oracle.amax(x).view(np.uint32)
    r = nv.quantize(xd, nv.AXIS_COLS, nv.MODE_4OVER6, nv.RULE_MSE)
    assert r["gscale"].cpu().numpy()[0].view(np.uint32) == g_ref.view(np.uint32)


def test_large_rowwise_sampled_rows(big):
    x, xd, g_ref = big
    banner("row-wise quantize across segment seams")
    r = nv.quantize(xd, nv.AXIS_COLS, nv.MODE_4OVER6, nv.RULE_MSE, selmap=True)
    torch.cuda.synchronize()
    pick = sample_rows()
    ref = oracle.quantize(x[pick], nv.AXIS_COLS, nv.MODE_4OVER6, nv.RULE_MSE, gscale=g_ref,
                          want_err=False)
    np.testing.assert_array_equal(r["packed"][torch.from_numpy(pick).cuda()].cpu().numpy()
                                  .reshape(-1), ref["packed"])
    np.testing.assert_array_equal(r["scales"][torch.from_numpy(pick).cuda()].cpu().numpy()
                                  .reshape(-1), ref["scales"])
    bpr = COLS // 16
    bits = np.unpackbits(r["selmap"].cpu().numpy(), bitorder="little")[: ROWS * bpr]
    want = np.unpackbits(ref["selmap"], bitorder="little")[: pick.size * bpr]
    np.testing.assert_array_equal(bits.reshape(ROWS, bpr)[pick].reshape(-1), want)

    banner("dequantize across segment seams")
    out = nv.dequantize(r["packed"], r["scales"], r["gscale"], ROWS, COLS, nv.AXIS_COLS,
                        torch.bfloat16)
    got = out[torch.from_numpy(pick).cuda()].view(torch.int16).cpu().numpy()
    deq = oracle.dequantize(ref["packed"], ref["scales"], g_ref, pick.size, COLS, nv.AXIS_COLS,
                            out_bf16=True)
    np.testing.assert_array_equal(got, deq.view(np.int16))
    del out, r


def test_large_column_blocked_sampled_columns(big):
    x, xd, _ = big
    rows, cols = COLS, ROWS  # the same bytes viewed as 16384 x 65600
    xv = x.reshape(rows, cols)
    banner(f"column-blocked {rows}x{cols}")
    g_ref = oracle.global_scale(oracle.amax(xv), nv.MODE_4OVER6)
    r = nv.quantize(xd.view(rows, cols), nv.AXIS_ROWS, nv.MODE_4OVER6, nv.RULE_MAE)
    torch.cuda.synchronize()
    assert r["gscale"].cpu().numpy()[0].view(np.uint32) == g_ref.view(np.uint32)
    rng = np.random.default_rng(4)
    pick = np.unique(np.concatenate([[0, 63, 64, cols - 1], rng.integers(0, cols, 12)]))
    ref = oracle.quantize(np.ascontiguousarray(xv[:, pick]), nv.AXIS_ROWS, nv.MODE_4OVER6,
                          nv.RULE_MAE, gscale=g_ref, want_selmap=False, want_err=False)
    idx = torch.from_numpy(pick).cuda()
    np.testing.assert_array_equal(r["packed"][idx].cpu().numpy().reshape(-1), ref["packed"])
    np.testing.assert_array_equal(r["scales"][idx].cpu().numpy().reshape(-1), ref["scales"])
    del r


# ------------------------------------------------ outlier-channel path ----

RES_ROWS, RES_COLS, RES_NRES = 140000, 8192, 512  # 2.3 GB of bf16: offsets past 2^31 bytes


@pytest.fixture(scope="module")
def big_res():
    banner(f"generating {RES_ROWS}x{RES_COLS}")
    x = testkit.fill((RES_ROWS, RES_COLS), testkit.STUDENT_T3, 0.5, 0x7E5)
    testkit.scale_columns(x, testkit.sample(0x7E6, RES_COLS, 16), 40.0)
    xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    yield x, xd
    del xd
    torch.cuda.empty_cache()


def test_large_channel_order(big_res):
    """Column maxima over 2.3 GB (the absmax pass splits its rows below 2^31
    bytes per workgroup range) against numpy, in row chunks."""
    x, xd = big_res
    banner("channel maxima and order over 2.3 GB")
    absmax, perm = nv.channel_order(xd)
    got = absmax.cpu().numpy()
    want = np.zeros(RES_COLS, np.float32)
    for r0 in range(0, RES_ROWS, 8192):
        want = np.maximum(want, np.abs(testkit.bf16_to_f32(x[r0:r0 + 8192])).max(axis=0))
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))
    np.testing.assert_array_equal(perm.cpu().numpy(), oracle.channel_order(want))


def test_large_residual_sampled_rows(big_res):
    """Two-stage quantize of rows past 2^31 input bytes (64-bit row offsets in
    the per-wave kernel), sampled rows against the oracle with the same g."""
    x, xd = big_res
    banner("residual quantize over 2.3 GB")
    rng = np.random.default_rng(8)
    perm = rng.permutation(RES_COLS).astype(np.int32)
    r = nv.quantize_residual(xd, torch.from_numpy(perm).cuda(), RES_NRES)
    torch.cuda.synchronize()
    g = np.float32(r["gscale"].cpu().numpy()[0])
    assert g.view(np.uint32) == oracle.global_scale(oracle.amax(x), nv.MODE_4OVER6).view(np.uint32)
    pick = np.unique(np.concatenate([[0, 131071, 131072, RES_ROWS - 1],
                                     rng.integers(0, RES_ROWS, 28)]))
    ref = oracle.quantize_residual(x[pick], perm, RES_NRES, nv.MODE_4OVER6, nv.RULE_MSE, gscale=g)
    idx = torch.from_numpy(pick).cuda()
    np.testing.assert_array_equal(r["packed"][idx].cpu().numpy(), ref["packed"])
    np.testing.assert_array_equal(r["scales"][idx].cpu().numpy(), ref["scales"])
    del r


WIDE_ROWS, WIDE_COLS, WIDE_NRES = 70000, 16384, 512  # 2.3 GB: rows start past 2^31 bytes


def test_large_rmsnorm_residual_wide_sampled_rows():
    """The fused RMSNorm path on rows of 16384 channels (the workgroup-shared
    kernel) over 2.3 GB with a given g: rows on both sides of the 2^31-byte
    seam and random rows against the oracle's RMSNorm and two-stage quantize."""
    banner(f"rmsnorm+residual {WIDE_ROWS}x{WIDE_COLS}")
    x = testkit.fill((WIDE_ROWS, WIDE_COLS), testkit.STUDENT_T3, 0.5, 0x71D)
    w = testkit.fill((WIDE_COLS,), testkit.NORMAL, 1.0, 0x71E)
    xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    wd = torch.from_numpy(w.view(np.int16)).cuda().view(torch.bfloat16)
    rng = np.random.default_rng(0x71F)
    perm = rng.permutation(WIDE_COLS).astype(np.int32)
    g = np.float32(0.004)
    gd = torch.tensor([float(g)], dtype=torch.float32, device="cuda")
    r = nv.rmsnorm_quantize_residual(xd, torch.from_numpy(perm).cuda(), WIDE_NRES, weight=wd,
                                     eps=1e-6, gscale=gd)
    torch.cuda.synchronize()
    seam = (1 << 31) // (WIDE_COLS * 2)  # first row starting at or past 2^31 bytes
    pick = np.unique(np.concatenate([[0, seam - 1, seam, seam + 1, WIDE_ROWS - 1],
                                     rng.integers(0, WIDE_ROWS, 27)]))
    y = oracle.rmsnorm(x[pick], w, 1e-6)
    ref = oracle.quantize_residual(y, perm, WIDE_NRES, nv.MODE_4OVER6, nv.RULE_MSE, gscale=g)
    idx = torch.from_numpy(pick).cuda()
    np.testing.assert_array_equal(r["packed"][idx].cpu().numpy(), ref["packed"])
    np.testing.assert_array_equal(r["scales"][idx].cpu().numpy(), ref["scales"])
    del r, xd


def test_large_w4a4_product_sampled_rows():
    """An activation operand of 2.25 GB of codes: the tiles' base addresses
    pass 2^31 bytes (64-bit per-tile bases, 32-bit offsets within a tile);
    sampled rows (first and last tiles among them) against the oracle."""
    M, N, K = 1_100_000, 48, 4096
    banner(f"W4A4 product {M}x{N}x{K}")
    rng = np.random.default_rng(0xA4)
    pa = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    sa = rng.integers(0x30, 0x48, (M, K // 16), dtype=np.uint8)
    pb = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    sb = rng.integers(0x30, 0x48, (N, K // 16), dtype=np.uint8)
    ga, gb = np.float32(0.01), np.float32(0.02)
    a = {"packed": torch.from_numpy(pa).cuda(), "scales": torch.from_numpy(sa).cuda(),
         "gscale": torch.tensor([float(ga)], device="cuda")}
    b = {"packed": torch.from_numpy(pb).cuda(), "scales": torch.from_numpy(sb).cuda(),
         "gscale": torch.tensor([float(gb)], device="cuda")}
    y = nv.gemm(a, b)
    torch.cuda.synchronize()
    rows = np.concatenate([[0, 255, 256, M // 2, M - 257, M - 1],
                           rng.choice(M, 42, replace=False)])
    got = y[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    want, gabs = oracle.gemm(pa[rows], sa[rows], ga, pb, sb, gb, len(rows), N, K, want_abs=True)
    tol = (K + K // 16 + 2) * 2.0 ** -23 * gabs + 2.0 ** -126
    assert np.all(np.abs(got - want) <= tol)
    del a, b, y
    torch.cuda.empty_cache()
