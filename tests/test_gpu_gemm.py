"""GPU parity of the W4A4 product (nvfp4_gemm): out = ga * gb * sum_k a b for
NVFP4 activations and weights blocked along K ("Why Gated DeltaNet in hybrid
27B LLMs withstands 4-bit quantization", 'Background'; the augmented product
over K_in + S of the "ARCQuant" summary, 'Methodology').

The operands decode exactly and their products are exact in fp32, so the
only difference from the oracle's binary64 sum is the fp32 accumulation and
the final scaling.  The tests use the bound the header states,
|out - exact| <= (K + K/16 + 2) * 2^-23 * ga * gb * sum |a b|, and are
bit-exact where every partial sum is representable (unit scales, g = 1).
Shapes cover ragged tile edges in M and N, K tails that are not a multiple
of the 128-wide stage, one block, both tile widths (256 x 128 for small
products, 256 x 256 for large ones), and the
32768 x 5120 x 5120 prefill product at full size (sampled rows and columns
against the oracle)."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_wave64_amd as nv
import oracle
import testkit
from tests._parity import Guarded, to_device

pytestmark = pytest.mark.gpu

F46, STD, MSE = nv.MODE_4OVER6, nv.MODE_STD, nv.RULE_MSE


def banner(msg):
    print(f"\n[gpu-gemm] {msg}", flush=True)


def random_nvfp4(seed, rows, K, scale_lo=0x00, scale_hi=0x7E):
    """Seeded random codes and E4M3 scale bytes (the NaN byte excluded)."""
    rng = np.random.default_rng(seed)
    packed = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    scales = rng.integers(scale_lo, scale_hi + 1, (rows, K // 16), dtype=np.uint8)
    return packed, scales


def dev_operand(packed, scales, g):
    return {"packed": torch.from_numpy(np.ascontiguousarray(packed)).cuda(),
            "scales": torch.from_numpy(np.ascontiguousarray(scales)).cuda(),
            "gscale": torch.tensor([float(np.float32(g))], dtype=torch.float32, device="cuda")}


def gpu_gemm(pa, sa, ga, pb, sb, gb, out_dtype=torch.float32):
    M, N = pa.shape[0], pb.shape[0]
    esz = 4 if out_dtype == torch.float32 else 2
    buf = Guarded(M * N * esz, out_dtype)
    nv.gemm(dev_operand(pa, sa, ga), dev_operand(pb, sb, gb), out_dtype, out=buf.view)
    torch.cuda.synchronize()
    buf.check()
    return buf.view.float().cpu().numpy().astype(np.float64).reshape(M, N)


def shifted(scales, off):
    """Device copy of a scale tensor starting `off` bytes past an allocation's
    start (the bytes before it hold 0x7E)."""
    big = torch.full((scales.size + off,), 0x7E, dtype=torch.uint8, device="cuda")
    t = big[off:]
    t.copy_(torch.from_numpy(np.ascontiguousarray(scales).reshape(-1)).cuda())
    return t.view(scales.shape)


def tile_shape(M, N, splits=1):
    """The tile shape the library picks (its documented rule): rounds of
    tiles, one per compute unit, times 43, 61 or 100 for 128 x 128, 256 x 128
    and 256 x 256 tiles; the cheapest wins, ties to the larger tile."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count

    def cost(tm, tn, w):
        units = -(-M // tm) * -(-N // tn) * splits
        return -(-units // cus) * w

    small, narrow, wide = cost(128, 128, 43), cost(256, 128, 61), cost(256, 256, 100)
    if small < narrow and small < wide:
        return "128x128"
    return "256x128" if narrow < wide else "256x256"


def bound(K, gabs):
    return (K + K // 16 + 2) * 2.0 ** -23 * gabs + 2.0 ** -126


def assert_within(got, want, gabs, K, extra_rel=0.0, what=""):
    err = np.abs(got - want)
    tol = bound(K, gabs) + extra_rel * np.abs(want)
    bad = np.argwhere(err > tol)
    assert bad.size == 0, (what, bad[:5].tolist(), got[tuple(bad[0])], want[tuple(bad[0])])


SHAPES = [(1, 1, 16), (31, 17, 48), (32, 32, 64), (256, 256, 64), (257, 255, 80),
          (300, 270, 320), (513, 259, 336), (1000, 700, 1040), (64, 640, 5120),
          (200, 96, 5376)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_unit_scales_are_bit_exact(M, N, K):
    banner(f"unit scales {M}x{N}x{K}")
    pa, _ = random_nvfp4(M * 7 + K, M, K)
    pb, _ = random_nvfp4(N * 11 + K, N, K)
    sa = np.full((M, K // 16), 0x38, np.uint8)  # E4M3 1.0
    sb = np.full((N, K // 16), 0x38, np.uint8)
    got = gpu_gemm(pa, sa, 1.0, pb, sb, 1.0)
    want = oracle.gemm(pa, sa, 1.0, pb, sb, 1.0, M, N, K)
    # Every partial sum is a multiple of 1/4 below 2^22: exact in fp32.
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_random_operands_within_the_bound(M, N, K, out_dtype):
    banner(f"random operands {M}x{N}x{K} {out_dtype}")
    pa, sa = random_nvfp4(M + 3 * K, M, K)
    pb, sb = random_nvfp4(N + 5 * K + 1, N, K)
    ga, gb = np.float32(0.37), np.float32(1.9e-3)
    got = gpu_gemm(pa, sa, ga, pb, sb, gb, out_dtype)
    want, gabs = oracle.gemm(pa, sa, ga, pb, sb, gb, M, N, K, want_abs=True)
    extra = 2.0 ** -8 if out_dtype == torch.bfloat16 else 0.0
    assert_within(got, want, gabs, K, extra, f"{M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,off_a,off_b", [(70, 90, 320, 1, 3), (257, 33, 336, 2, 1),
                                                (31, 300, 1040, 3, 0)])
def test_scale_tensors_not_four_byte_aligned(M, N, K, off_a, off_b):
    """Scale bytes may start anywhere: each tile's scale window is read from
    the 4-byte boundary below its first byte."""
    banner(f"scale pointers offset by {off_a}, {off_b} bytes ({M}x{N}x{K})")
    pa, sa = random_nvfp4(M + K + off_a, M, K)
    pb, sb = random_nvfp4(N + K + off_b, N, K)
    a = dev_operand(pa, sa, 0.5)
    b = dev_operand(pb, sb, 0.25)
    a["scales"] = shifted(sa, off_a)
    b["scales"] = shifted(sb, off_b)
    got = nv.gemm(a, b).cpu().numpy().astype(np.float64)
    want, gabs = oracle.gemm(pa, sa, 0.5, pb, sb, 0.25, M, N, K, want_abs=True)
    assert_within(got, want, gabs, K)


def test_bf16_output_at_a_two_byte_offset():
    banner("bf16 output not 4-byte aligned")
    M, N, K = 70, 64, 96
    pa, sa = random_nvfp4(43, M, K)
    pb, sb = random_nvfp4(44, N, K)
    big = torch.zeros(M * N + 1, dtype=torch.bfloat16, device="cuda")
    out = big[1:]  # data pointer 2 bytes past an aligned one
    nv.gemm(dev_operand(pa, sa, 0.5), dev_operand(pb, sb, 0.25), torch.bfloat16, out=out)
    ref = gpu_gemm(pa, sa, 0.5, pb, sb, 0.25, torch.bfloat16)
    torch.cuda.synchronize()
    assert big[0].item() == 0.0
    np.testing.assert_array_equal(out.float().cpu().numpy().astype(np.float64).reshape(M, N), ref)


def test_bf16_output_is_the_rounded_fp32_output():
    banner("bf16 = RNE(fp32)")
    M, N, K = 300, 270, 336
    pa, sa = random_nvfp4(41, M, K)
    pb, sb = random_nvfp4(42, N, K)
    f = gpu_gemm(pa, sa, 0.5, pb, sb, 0.25, torch.float32)
    b = gpu_gemm(pa, sa, 0.5, pb, sb, 0.25, torch.bfloat16)
    want = torch.from_numpy(f.astype(np.float32)).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(b, want.astype(np.float64))


@pytest.mark.parametrize("mode", [STD, F46])
def test_quantized_activations_and_weights(mode):
    banner(f"quantized X W^T mode={mode}")
    M, N, K = 384, 320, 1024
    x = testkit.fill((M, K), testkit.STUDENT_T3, 0.5, 51)
    testkit.scale_columns(x, testkit.sample(52, K, 8), 100.0)
    w = testkit.fill((N, K), testkit.NORMAL, 0.02, 53)
    qx = oracle.quantize(x, nv.AXIS_COLS, mode, MSE, want_selmap=False, want_err=False)
    qw = oracle.quantize(w, nv.AXIS_COLS, mode, MSE, want_selmap=False, want_err=False)
    shp = lambda q, r: (q["packed"].reshape(r, K // 2), q["scales"].reshape(r, K // 16))
    pa, sa = shp(qx, M)
    pb, sb = shp(qw, N)
    got = gpu_gemm(pa, sa, qx["gscale"], pb, sb, qw["gscale"])
    want, gabs = oracle.gemm(pa, sa, qx["gscale"], pb, sb, qw["gscale"], M, N, K, want_abs=True)
    assert_within(got, want, gabs, K)


@pytest.mark.parametrize("mode", [STD, F46])
def test_augmented_product(mode):
    banner(f"augmented product mode={mode}")
    M, N, K, S = 256, 192, 2048, 128
    x = testkit.fill((M, K), testkit.STUDENT_T3, 0.5, 61)
    testkit.scale_columns(x, testkit.sample(62, K, 16), 60.0)
    w = testkit.fill((N, K), testkit.NORMAL, 0.02, 63)
    perm = oracle.channel_order(oracle.channel_absmax(x))
    qa = oracle.quantize_residual(x, perm, S, mode, MSE)
    qb = oracle.quantize_residual(w, perm, S, mode, MSE, duplicate=True)
    # The weight side through the library matches the oracle bit for bit.
    bufs = {"packed": Guarded(N * (K + S) // 2), "scales": Guarded(N * (K + S) // 16),
            "gscale": Guarded(4, torch.float32)}
    pd = torch.from_numpy(np.ascontiguousarray(perm, np.int32)).cuda()
    nv.quantize_residual(to_device(w), pd, S, mode, MSE, out={k: b.view for k, b in bufs.items()},
                         duplicate=True)
    torch.cuda.synchronize()
    for b in bufs.values():
        b.check()
    np.testing.assert_array_equal(bufs["packed"].view.cpu().numpy(), qb["packed"].reshape(-1))
    np.testing.assert_array_equal(bufs["scales"].view.cpu().numpy(), qb["scales"].reshape(-1))
    assert bufs["gscale"].view.cpu().numpy()[0] == qb["gscale"]
    got = gpu_gemm(qa["packed"], qa["scales"], qa["gscale"], qb["packed"], qb["scales"],
                   qb["gscale"])
    want, gabs = oracle.gemm(qa["packed"], qa["scales"], qa["gscale"], qb["packed"],
                             qb["scales"], qb["gscale"], M, N, K + S, want_abs=True)
    assert_within(got, want, gabs, K + S)


def test_full_size_prefill_product_sampled():
    M, N, K = 32768, 5120, 5120
    banner(f"full size {M}x{N}x{K}")
    pa, sa = random_nvfp4(71, M, K, 0x28, 0x50)
    pb, sb = random_nvfp4(72, N, K, 0x28, 0x50)
    ga, gb = np.float32(2.5e-3), np.float32(4.0e-5)
    got = gpu_gemm(pa, sa, ga, pb, sb, gb)
    rng = np.random.default_rng(73)
    rows = np.concatenate([[0, 255, 256, M - 1], rng.choice(M, 44, replace=False)])
    cols = np.concatenate([[0, 127, 128, N - 1], rng.choice(N, 44, replace=False)])
    want, gabs = oracle.gemm(pa[rows], sa[rows], ga, pb[cols], sb[cols], gb, len(rows), len(cols),
                             K, want_abs=True)
    assert_within(got[np.ix_(rows, cols)], want, gabs, K, what="sampled")
    assert np.isfinite(got).all()


@pytest.mark.parametrize("shape", ["256x256", "256x128"])
@pytest.mark.parametrize("K,off", [(592, 0), (640, 1)])
def test_large_tiles_with_ragged_edges(K, off, shape):
    # The tile shape follows from how many rounds of tiles (one per compute
    # unit) each shape needs; the small shapes elsewhere in this file take
    # 128 x 128 tiles.  These take 256 x 256 tiles (one round of them, where
    # 256 x 128 tiles need two) or 256 x 128 tiles (one round, where 128 x 128
    # ones need two) on any device, with M and N ending mid-tile and K ending
    # mid-stage (592) or scale tensors off the 4-byte grid (640 with an
    # offset): all rows of the last tile row and a sample of the others,
    # against the oracle over every column.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if shape == "256x256":
        tiles_n = 17
        tiles_m = cus // tiles_n
        M, N = 256 * tiles_m - 37, 256 * tiles_n - 100
    else:
        tiles_m = max(1, cus // 40)
        M, N = 256 * tiles_m - 37, 128 * 40 - 100
    assert tile_shape(M, N) == shape, (M, N, cus)
    banner(f"{shape} tiles {M}x{N}x{K} scale offset {off}")
    pa, sa = random_nvfp4(131 + K, M, K, 0x28, 0x50)
    pb, sb = random_nvfp4(132 + K, N, K, 0x28, 0x50)
    ga, gb = np.float32(3.0e-2), np.float32(7.0e-4)
    a, b = dev_operand(pa, sa, ga), dev_operand(pb, sb, gb)
    a["scales"], b["scales"] = shifted(sa, off), shifted(sb, off)
    buf = Guarded(M * N * 4, torch.float32)
    nv.gemm(a, b, torch.float32, out=buf.view)
    torch.cuda.synchronize()
    buf.check()
    got = buf.view.cpu().numpy().astype(np.float64).reshape(M, N)
    rng = np.random.default_rng(133)
    rows = np.unique(np.concatenate([np.arange(256 * (tiles_m - 1), M), [0, 127, 128, 255, 256],
                                     rng.choice(M, 24, replace=False)]))
    want, gabs = oracle.gemm(pa[rows], sa[rows], ga, pb, sb, gb, len(rows), N, K, want_abs=True)
    assert_within(got[rows], want, gabs, K, what="wide tiles")
    assert np.isfinite(got).all()


def test_tile_width_does_not_change_results():
    # Every tile shape gives every output the same summation order (the same
    # stages and MFMA steps, in order), so the first rows of products that
    # take 128 x 128 and 256 x 128 tiles equal, bit for bit, those rows of a
    # product large enough for 256 x 256 tiles.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    N, K = 5120, 1040
    M_narrow = 256 * max(1, cus // 64)
    M_big = 256 * -(-4 * cus // 20)
    assert tile_shape(128, N) == "128x128", cus
    assert tile_shape(M_narrow, N) == "256x128", (cus, M_narrow)
    assert tile_shape(M_big, N) == "256x256", (cus, M_big)
    banner(f"tile shapes agree: 128, {M_narrow} vs {M_big} rows, {N}x{K}")
    pa, sa = random_nvfp4(141, M_big, K, 0x28, 0x50)
    pb, sb = random_nvfp4(142, N, K, 0x28, 0x50)
    small = gpu_gemm(pa[:M_narrow], sa[:M_narrow], 0.75, pb, sb, 1.0e-3)
    tiny = gpu_gemm(pa[:128], sa[:128], 0.75, pb, sb, 1.0e-3)
    big = gpu_gemm(pa, sa, 0.75, pb, sb, 1.0e-3)
    np.testing.assert_array_equal(small, big[:M_narrow])
    np.testing.assert_array_equal(tiny, big[:128])
    want, gabs = oracle.gemm(pa[:128], sa[:128], 0.75, pb, sb, 1.0e-3, 128, N, K, want_abs=True)
    assert_within(tiny, want, gabs, K)


def test_long_k_errors_are_far_inside_the_bound():
    # 512 stages of the K loop.  The bound is a worst case (every rounding
    # in the same direction); random-sign sums grow like sqrt(K), so the
    # typical error must sit well inside it.
    M, N, K = 48, 32, 65536
    banner(f"long K {M}x{N}x{K}")
    pa, sa = random_nvfp4(91, M, K, 0x30, 0x48)
    pb, sb = random_nvfp4(92, N, K, 0x30, 0x48)
    got = gpu_gemm(pa, sa, 0.125, pb, sb, 0.5)
    want, gabs = oracle.gemm(pa, sa, 0.125, pb, sb, 0.5, M, N, K, want_abs=True)
    assert_within(got, want, gabs, K)
    ratio = np.abs(got - want) / bound(K, gabs)
    assert ratio.mean() < 0.01 and ratio.max() < 0.1, (ratio.mean(), ratio.max())


def test_deterministic_and_exact_scalings():
    banner("determinism, g scaling, zero g")
    M, N, K = 257, 255, 1040
    pa, sa = random_nvfp4(81, M, K)
    pb, sb = random_nvfp4(82, N, K)
    a = gpu_gemm(pa, sa, 0.75, pb, sb, 0.5)
    np.testing.assert_array_equal(a, gpu_gemm(pa, sa, 0.75, pb, sb, 0.5))
    # Scaling ga by 4 scales RN(ga * gb) and every output by 4 exactly.
    np.testing.assert_array_equal(gpu_gemm(pa, sa, 3.0, pb, sb, 0.5), 4.0 * a)
    # Swapping the operands transposes the product (same terms, same order
    # within each 16-wide step is not guaranteed, so within the bound).
    t = gpu_gemm(pb, sb, 0.5, pa, sa, 0.75)
    want, gabs = oracle.gemm(pa, sa, 0.75, pb, sb, 0.5, M, N, K, want_abs=True)
    assert_within(t.T, want, gabs, K)
    z = gpu_gemm(pa, sa, 0.0, pb, sb, 0.5)
    assert (z == 0).all()


def test_forward_and_backward_products_from_one_dual_quantization():
    """4/6 on weights and gradients: one nvfp4_quantize_dual call on a
    weight W [N][K] gives the row-blocked operand of the forward product
    Y = X W^T (reduction over K) and the column-blocked one, the layout of
    W^T [K][N] blocked along N, of the backward product dX = dY W
    (reduction over N).  Both products against the oracle on the same
    operands, within the bound."""
    banner("forward and backward products from one dual quantization")
    M, N, K = 192, 160, 320
    w = testkit.fill((N, K), testkit.NORMAL, 0.02, 101)
    x = testkit.fill((M, K), testkit.STUDENT_T3, 0.5, 102)
    dy = testkit.fill((M, N), testkit.NORMAL, 1e-3, 103)
    qd = nv.quantize_dual(to_device(w), F46, MSE)
    qx = nv.quantize(to_device(x), nv.AXIS_COLS, F46, MSE)
    qdy = nv.quantize(to_device(dy), nv.AXIS_COLS, F46, MSE)
    g = qd["gscale"]
    w_rows = {"packed": qd["rows"]["packed"].view(N, K // 2),
              "scales": qd["rows"]["scales"].view(N, K // 16), "gscale": g}
    w_cols = {"packed": qd["cols"]["packed"].view(K, N // 2),
              "scales": qd["cols"]["scales"].view(K, N // 16), "gscale": g}
    a_x = {"packed": qx["packed"].view(M, K // 2), "scales": qx["scales"].view(M, K // 16),
           "gscale": qx["gscale"]}
    a_dy = {"packed": qdy["packed"].view(M, N // 2), "scales": qdy["scales"].view(M, N // 16),
            "gscale": qdy["gscale"]}
    y = nv.gemm(a_x, w_rows).cpu().numpy().astype(np.float64)
    dx = nv.gemm(a_dy, w_cols).cpu().numpy().astype(np.float64)
    # The oracle's own quantizations of the same tensors (both layouts of W).
    ow = oracle.quantize(w, nv.AXIS_COLS, F46, MSE, want_selmap=False, want_err=False)
    owt = oracle.quantize(w, nv.AXIS_ROWS, F46, MSE, want_selmap=False, want_err=False)
    ox = oracle.quantize(x, nv.AXIS_COLS, F46, MSE, want_selmap=False, want_err=False)
    ody = oracle.quantize(dy, nv.AXIS_COLS, F46, MSE, want_selmap=False, want_err=False)
    assert owt["gscale"] == ow["gscale"] == np.float32(g.item())
    want_y, gy = oracle.gemm(ox["packed"], ox["scales"], ox["gscale"], ow["packed"], ow["scales"],
                             ow["gscale"], M, N, K, want_abs=True)
    want_dx, gdx = oracle.gemm(ody["packed"], ody["scales"], ody["gscale"], owt["packed"],
                               owt["scales"], owt["gscale"], M, K, N, want_abs=True)
    assert_within(y, want_y, gy, K, what="forward")
    assert_within(dx, want_dx, gdx, N, what="backward")
    # And both approximate the bf16 products.
    xf, wf = testkit.bf16_to_f32(x).astype(np.float64), testkit.bf16_to_f32(w).astype(np.float64)
    dyf = testkit.bf16_to_f32(dy).astype(np.float64)
    for got, exact in ((y, xf @ wf.T), (dx, dyf @ wf)):
        rel = np.linalg.norm(got - exact) / np.linalg.norm(exact)
        assert rel < 0.2, rel


# ---- nvfp4_gemm_splitk: the same product with K split into ranges ----

def gpu_gemm_split(pa, sa, ga, pb, sb, gb, splits, out_dtype=torch.float32, ws=None):
    """Split product through the C ABI with guarded output and workspace."""
    M, N = pa.shape[0], pb.shape[0]
    esz = 4 if out_dtype == torch.float32 else 2
    buf = Guarded(M * N * esz, out_dtype)
    wsb = ws if ws is not None else Guarded(splits * M * N * 4, torch.float32)
    nv.gemm(dev_operand(pa, sa, ga), dev_operand(pb, sb, gb), out_dtype, out=buf.view,
            splits=splits, workspace=wsb.view)
    torch.cuda.synchronize()
    buf.check()
    wsb.check()
    return buf.view.float().cpu().numpy().astype(np.float64).reshape(M, N)


SPLIT_SHAPES = [(31, 17, 272), (256, 300, 1040), (257, 129, 5120), (128, 640, 5376)]


@pytest.mark.parametrize("M,N,K", SPLIT_SHAPES)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_one_split_equals_the_unsplit_product(M, N, K, out_dtype):
    banner(f"split 1 vs unsplit {M}x{N}x{K} {out_dtype}")
    pa, sa = random_nvfp4(M + 7 * K, M, K)
    pb, sb = random_nvfp4(N + 9 * K, N, K)
    got = gpu_gemm_split(pa, sa, 0.37, pb, sb, 1.9e-3, 1, out_dtype)
    want = gpu_gemm(pa, sa, 0.37, pb, sb, 1.9e-3, out_dtype)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("M,N,K", SPLIT_SHAPES)
def test_split_products_within_the_bound(M, N, K):
    nchunks = -(-K // 128)
    pa, sa = random_nvfp4(M + 11 * K, M, K)
    pb, sb = random_nvfp4(N + 13 * K, N, K)
    ga, gb = np.float32(0.37), np.float32(1.9e-3)
    want, gabs = oracle.gemm(pa, sa, ga, pb, sb, gb, M, N, K, want_abs=True)
    for splits in sorted({2, 3, 7, nchunks} & set(range(1, min(64, nchunks) + 1))):
        banner(f"{splits} splits {M}x{N}x{K}")
        got = gpu_gemm_split(pa, sa, ga, pb, sb, gb, splits)
        assert_within(got, want, gabs, K, what=f"{splits} splits")
        again = gpu_gemm_split(pa, sa, ga, pb, sb, gb, splits)
        np.testing.assert_array_equal(got, again)


@pytest.mark.parametrize("splits", [2, 5])
def test_split_unit_scales_are_bit_exact(splits):
    M, N, K = 200, 96, 1296  # 11 chunks of K, the last one partial
    banner(f"unit scales, {splits} splits {M}x{N}x{K}")
    pa, _ = random_nvfp4(301, M, K)
    pb, _ = random_nvfp4(302, N, K)
    sa = np.full((M, K // 16), 0x38, np.uint8)
    sb = np.full((N, K // 16), 0x38, np.uint8)
    got = gpu_gemm_split(pa, sa, 1.0, pb, sb, 1.0, splits)
    np.testing.assert_array_equal(got, oracle.gemm(pa, sa, 1.0, pb, sb, 1.0, M, N, K))


def test_split_workspace_reused_by_a_smaller_product():
    # The workspace holds the previous call's sums on entry; a second,
    # smaller call with the same workspace must not depend on them.
    ws = Guarded(4 * 300 * 200 * 4, torch.float32)
    for (M, N, K, splits) in [(300, 200, 2048, 4), (70, 90, 640, 3)]:
        banner(f"workspace reuse {M}x{N}x{K}, {splits} splits")
        pa, sa = random_nvfp4(M + K, M, K)
        pb, sb = random_nvfp4(N + K, N, K)
        got = gpu_gemm_split(pa, sa, 0.5, pb, sb, 0.25, splits, ws=ws)
        want, gabs = oracle.gemm(pa, sa, 0.5, pb, sb, 0.25, M, N, K, want_abs=True)
        assert_within(got, want, gabs, K)


def test_decode_sized_product_with_the_hinted_split():
    M, N, K = 128, 5120, 5120
    hint = nv.gemm_splits_hint(M, N, K)
    assert 2 <= hint <= K // 128 // 4, hint
    banner(f"decode-sized {M}x{N}x{K}, hint {hint}")
    pa, sa = random_nvfp4(401, M, K, 0x28, 0x50)
    pb, sb = random_nvfp4(402, N, K, 0x28, 0x50)
    ga, gb = np.float32(2.5e-3), np.float32(4.0e-5)
    a, b = dev_operand(pa, sa, ga), dev_operand(pb, sb, gb)
    got = nv.gemm(a, b, torch.float32, splits="auto").cpu().numpy().astype(np.float64)
    cols = np.concatenate([[0, 127, 128, N - 1], np.random.default_rng(403).choice(N, 60, False)])
    want, gabs = oracle.gemm(pa, sa, ga, pb[cols], sb[cols], gb, M, len(cols), K, want_abs=True)
    assert_within(got[:, cols], want, gabs, K)
    assert nv.gemm_splits_hint(32768, 5120, 5120) == 1
    assert nv.gemm_splits_hint(128, 5120, 256) == 1


def test_split_reduce_vector_and_scalar_paths_agree():
    # mn a multiple of 4 with aligned buffers takes the 16-byte reduce; a
    # bf16 output 2 bytes off its allocation takes the element-wise one.
    # Same split count, same sums: the outputs agree bit for bit.
    M, N, K, splits = 256, 300, 1040, 3
    banner(f"split reduce paths {M}x{N}x{K}, {splits} splits")
    pa, sa = random_nvfp4(501, M, K)
    pb, sb = random_nvfp4(502, N, K)
    a, b = dev_operand(pa, sa, 0.37), dev_operand(pb, sb, 1.9e-3)
    aligned = nv.gemm(a, b, torch.bfloat16, splits=splits)
    raw = torch.full((M * N + 1,), 7, dtype=torch.bfloat16, device="cuda")
    shifted_out = raw[1:].view(M, N)
    nv.gemm(a, b, torch.bfloat16, out=shifted_out, splits=splits)
    torch.cuda.synchronize()
    assert raw[0].item() == 7
    np.testing.assert_array_equal(aligned.float().cpu().numpy(), shifted_out.float().cpu().numpy())
