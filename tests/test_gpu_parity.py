"""GPU parity: the HIP path (through the C ABI) against the oracle, element by
element on the same seeded inputs.  Codes, scale bytes, global scale and the
selection bitmap must be bit-exact; the per-tensor error sum must agree to
1e-6 relative (binary64 sums in a different order).

Workloads follow the five benchmark workloads (testkit.WORKLOADS): full
size, and reduced/ragged shapes that span several tiles and leave a partial
tail."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_wave64_amd as nv
import oracle
import testkit
from tests._parity import check_against_oracle, gpu_quantize, to_device, assert_same

pytestmark = pytest.mark.gpu

AXIS_ROWS, AXIS_COLS = nv.AXIS_ROWS, nv.AXIS_COLS
STD, F46 = nv.MODE_STD, nv.MODE_4OVER6
MSE, MAE, MAXE = nv.RULE_MSE, nv.RULE_MAE, nv.RULE_MAX
RULES = [(STD, MSE), (F46, MSE), (F46, MAE), (F46, MAXE)]


def banner(msg):
    print(f"\n[gpu-parity] {msg}", flush=True)


# ------------------------------------------------------------ full size ----

@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_config_full_size(cid):
    cfg = testkit.WORKLOADS[cid]
    banner(f"config {cid} {cfg.name} {cfg.rows}x{cfg.cols}")
    x = testkit.make(cid)
    check_against_oracle(x, cfg.block_axis, cfg.mode, cfg.rule, what=f"config {cid}")


@pytest.mark.parametrize("axis", [AXIS_COLS, AXIS_ROWS])
def test_max_error_rule_full_size(axis):
    """The third selection rule of the method (minimum maximum error) on the
    4096 x 5120 activation workload, in both block layouts."""
    banner(f"max-error rule 4096x5120 axis={axis}")
    x = testkit.make(2)
    check_against_oracle(x, axis, F46, MAXE, what=f"max rule axis={axis}")


# ------------------------------------------------------------ ragged ----

RAGGED = [
    # (rows, cols): partial last chunk, several grid-stride iterations, one block
    (1, 16), (3, 48), (37, 5120), (129, 1040), (1000, 80), (2, 16 * 1001),
]


@pytest.mark.parametrize("rows,cols", RAGGED)
@pytest.mark.parametrize("mode,rule", RULES)
def test_rowwise_ragged(rows, cols, mode, rule):
    banner(f"rowwise {rows}x{cols} mode={mode} rule={rule}")
    x = testkit.fill((rows, cols), testkit.STUDENT_T3, 0.7, 1000 + rows * 7 + cols)
    check_against_oracle(x, AXIS_COLS, mode, rule, what=f"{rows}x{cols}")


RAGGED_COLS = [
    # (rows, cols): row blocks not a multiple of the 64-row tile, columns not
    # a multiple of the 64-column strip, columns not a multiple of 8
    (16, 1), (48, 70), (80, 64), (1040, 72), (256, 130), (16 * 37, 13), (2048, 200),
]


@pytest.mark.parametrize("rows,cols", RAGGED_COLS)
@pytest.mark.parametrize("mode,rule", RULES)
def test_colblocked_ragged(rows, cols, mode, rule):
    banner(f"colblocked {rows}x{cols} mode={mode} rule={rule}")
    x = testkit.fill((rows, cols), testkit.NORMAL, 1e-3, 2000 + rows * 3 + cols)
    testkit.scale_at(x.reshape(-1), testkit.sample(5, x.size, max(1, x.size // 100)), 30.0)
    check_against_oracle(x, AXIS_ROWS, mode, rule, what=f"{rows}x{cols}")


def test_colblocked_equals_rowwise_of_transpose():
    banner("colblocked vs rowwise of the transpose")
    x = testkit.make(5, rows=512, cols=384)
    a = gpu_quantize(x, AXIS_ROWS, F46, MAE)
    b = gpu_quantize(np.ascontiguousarray(x.T), AXIS_COLS, F46, MAE)
    for k in ("packed", "scales", "selmap"):
        np.testing.assert_array_equal(a[k], b[k])
    assert a["gscale"] == b["gscale"]


# ------------------------------------------------------------ edge cases ----

def test_all_zero_and_negative_zero():
    banner("zeros")
    x = np.zeros((4, 64), np.uint16)
    x[1, 5] = 0x8000
    x[3, 63] = 0x8000
    xc = np.zeros((32, 8), np.uint16)
    xc[17, 5] = 0x8000
    for mode, rule in RULES:
        gpu, _ = check_against_oracle(x, AXIS_COLS, mode, rule, what="zeros")
        assert gpu["gscale"] == 0 and gpu["err_sum"] == 0
        check_against_oracle(xc, AXIS_ROWS, mode, rule, what="zeros cols")


def test_extreme_magnitudes():
    banner("extremes")
    x = testkit.fill((8, 256), testkit.NORMAL, 1.0, 77)
    x[0, 0] = 0x7F7F  # bf16 max finite ~3.39e38
    x[1, :16] = np.arange(1, 17, dtype=np.uint16)  # bf16 subnormals
    x[2, 16:32] = 0x0080  # smallest normal
    for mode in (STD, F46):
        check_against_oracle(x, AXIS_COLS, mode, MSE, what="extremes")
    y = x.copy()
    y[0, 0] = 0x3F80  # make the subnormal rows matter relative to amax
    check_against_oracle(y, AXIS_COLS, F46, MAE, what="subnormal blocks")


def random_finite_patterns(shape, e_lo, e_hi, seed):
    """bf16 bit patterns with a random sign and mantissa and an exponent field
    drawn uniformly from [e_lo, e_hi] (0 gives zeros and subnormals; 255,
    infinity and NaN, is outside the contract and never drawn)."""
    rng = np.random.default_rng(seed)
    sign = rng.integers(0, 2, shape, dtype=np.uint16) << 15
    exp = rng.integers(e_lo, e_hi + 1, shape, dtype=np.uint16) << 7
    man = rng.integers(0, 128, shape, dtype=np.uint16)
    return (sign | exp | man).astype(np.uint16)


# Exponent windows: subnormal-heavy (amax near 1e-31), thirty binades
# around 1 (blocks spanning wide ranges), and the top of the range (amax
# near 3e38, squared errors overflowing to +inf).
PATTERN_WINDOWS = [(0, 24), (112, 142), (224, 254)]


@pytest.mark.parametrize("e_lo,e_hi", PATTERN_WINDOWS)
@pytest.mark.parametrize("mode,rule", RULES)
def test_random_finite_bit_patterns(e_lo, e_hi, mode, rule):
    """Whole tensors of random finite bf16 patterns in one exponent window,
    both block layouts, ragged shapes: every output bit-exact."""
    banner(f"random patterns e=[{e_lo},{e_hi}] mode={mode} rule={rule}")
    x = random_finite_patterns((96, 1040), e_lo, e_hi, 9000 + e_lo)
    _, ref = check_against_oracle(x, AXIS_COLS, mode, rule, what=f"patterns rows e>={e_lo}")
    xc = random_finite_patterns((272, 48), e_lo, e_hi, 9100 + e_lo)
    _, refc = check_against_oracle(xc, AXIS_ROWS, mode, rule, what=f"patterns cols e>={e_lo}")
    # Dequantize the oracle's outputs on the GPU, in both layouts and both
    # output types: decoded values range from subnormals to near 2^128.
    for axis, q, (rows, cols) in ((AXIS_COLS, ref, x.shape), (AXIS_ROWS, refc, xc.shape)):
        for dtype in (torch.float32, torch.bfloat16):
            want = oracle.dequantize(q["packed"], q["scales"], q["gscale"], rows, cols, axis,
                                     out_bf16=dtype == torch.bfloat16)
            out = nv.dequantize(torch.from_numpy(q["packed"]).cuda(),
                                torch.from_numpy(q["scales"]).cuda(),
                                torch.tensor([q["gscale"]], dtype=torch.float32, device="cuda"),
                                rows, cols, axis, dtype)
            got = out.view(torch.int16 if dtype == torch.bfloat16 else torch.int32).cpu().numpy()
            np.testing.assert_array_equal(got, want.view(got.dtype))


def test_tiny_tensor_amax():
    banner("tiny amax")
    x = np.zeros((2, 32), np.uint16)
    x[0, :4] = [0x0001, 0x8002, 0x0003, 0x0010]  # amax in the bf16 subnormal range
    for mode in (STD, F46):
        check_against_oracle(x, AXIS_COLS, mode, MSE, what="tiny amax")


def test_subnormal_and_zero_block_scales():
    banner("subnormal scales")
    rng = np.random.default_rng(4)
    f = (rng.standard_normal((64, 256)) * np.float32(10.0) ** rng.integers(-6, 1, (64, 16)).repeat(
        16, axis=1)).astype(np.float32)
    f[0, 0] = 1000.0
    x = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for mode, rule in RULES:
        gpu, ref = check_against_oracle(x, AXIS_COLS, mode, rule, what="subnormal scales")
    assert (ref["scales"] < 8).sum() > 10 and (ref["scales"] == 0).sum() > 10


def test_e2m1_midpoints_and_scale_ties():
    """Scaled values landing exactly on E2M1 midpoints (0.25, 0.75, ..., 5)
    and on E4M3 midpoints: with g = 1/6 (given) a block max of 6 has s6 = 6,
    and multiples of 1/2^k sit on the decision points."""
    banner("midpoints")
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32)
    vals = np.concatenate([mids, -mids, mids * 0.5, mids * 2.0])
    f = np.zeros((8, 64), np.float32)
    for r in range(8):
        f[r, :vals.size // 2] = np.roll(vals, r)[: vals.size // 2]
        f[r, 32:32 + vals.size // 2] = np.roll(vals, 3 * r)[vals.size // 2:]
    x = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for g in (1.0, 1.0 / 6, 0.5, 1.0 / 3, 2.0 ** -7):
        for mode, rule in RULES:
            check_against_oracle(x, AXIS_COLS, mode, rule, gscale=g, what=f"g={g}")


def test_given_scale_saturates():
    banner("given g saturation")
    x = testkit.fill((16, 512), testkit.STUDENT_T3, 3.0, 9)
    for g in (1e-3, 1e-6, 0.0):
        for mode in (STD, F46):
            check_against_oracle(x, AXIS_COLS, mode, MSE, gscale=g, what=f"g={g}")
            check_against_oracle(x, AXIS_ROWS, mode, MAE, gscale=g, what=f"cols g={g}")


def test_std_mode_bitmap_is_zero_and_err_is_sse():
    banner("std bitmap/err")
    x = testkit.make(1)
    gpu, ref = check_against_oracle(x, AXIS_COLS, STD, MAE, what="std")
    assert (gpu["selmap"] == 0).all()


def test_optional_outputs_absent():
    banner("no selmap / err")
    x = testkit.make(2, rows=64)
    for sel, err in [(False, False), (True, False), (False, True)]:
        check_against_oracle(x, AXIS_COLS, F46, MSE, selmap=sel, err=err, what=f"{sel},{err}")
        check_against_oracle(x, AXIS_ROWS, F46, MSE, selmap=sel, err=err, what=f"c {sel},{err}")


def test_deterministic_rerun():
    banner("determinism")
    x = testkit.make(4, rows=2048)
    a = gpu_quantize(x, AXIS_COLS, F46, MSE)
    b = gpu_quantize(x, AXIS_COLS, F46, MSE)
    for k in ("packed", "scales", "selmap"):
        np.testing.assert_array_equal(a[k], b[k])
    assert a["err_sum"] == pytest.approx(b["err_sum"], rel=1e-12)


def test_error_sum_accumulates_on_request():
    banner("err accumulate")
    x = testkit.make(2, rows=128)
    xd = to_device(x)
    ref = oracle.quantize(x, AXIS_COLS, F46, MSE)
    err = torch.full((1,), 5.0, dtype=torch.float64, device="cuda")
    r = nv.quantize(xd, AXIS_COLS, F46, MSE, err_sum=True, err_accumulate=True,
                    out={"err_sum": err})
    r = nv.quantize(xd, AXIS_COLS, F46, MSE, gscale=r["gscale"], err_sum=True,
                    err_accumulate=True, out={"err_sum": err})
    assert err.item() == pytest.approx(5.0 + 2 * ref["err_sum"], rel=1e-6)
    r = nv.quantize(xd, AXIS_COLS, F46, MSE, gscale=r["gscale"], err_sum=True,
                    out={"err_sum": err})  # without the flag the sum starts from zero
    assert err.item() == pytest.approx(ref["err_sum"], rel=1e-6)


def test_non_default_stream():
    banner("side stream")
    x = testkit.make(2, rows=256)
    s = torch.cuda.Stream()
    gpu = gpu_quantize(x, AXIS_COLS, F46, MSE, stream=s)
    ref = oracle.quantize(x, AXIS_COLS, F46, MSE)
    assert_same(gpu, ref, "side stream")


# ------------------------------------------------------------ amax / g ----

@pytest.mark.parametrize("n", [1, 7, 8, 9, 4097, 1 << 20, (1 << 20) + 5])
def test_amax_and_global_scale(n):
    banner(f"amax n={n}")
    x = testkit.fill((n,), testkit.STUDENT_T3, 2.0, n)
    xd = to_device(x)
    a = nv.amax(xd)
    want = oracle.amax(x)
    assert a.cpu().numpy()[0].view(np.uint32) == want.view(np.uint32)
    for mode in (STD, F46):
        g = nv.global_scale(a, mode)
        assert g.cpu().numpy()[0].view(np.uint32) == oracle.global_scale(want, mode).view(np.uint32)


# ------------------------------------------------------------ dequantize ----

@pytest.mark.parametrize("axis,shape", [(AXIS_COLS, (256, 1024)), (AXIS_ROWS, (256, 96)),
                                        (AXIS_COLS, (3, 48)), (AXIS_ROWS, (48, 5)),
                                        (AXIS_ROWS, (400, 200)), (AXIS_ROWS, (272, 130)),
                                        (AXIS_ROWS, (1040, 257))])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_dequantize_round_trip(axis, shape, dtype):
    banner(f"dequantize axis={axis} shape={shape} {dtype}")
    rows, cols = shape
    x = testkit.make(1, rows=rows, cols=cols)
    ref = oracle.quantize(x, axis, STD, MSE)
    want = oracle.dequantize(ref["packed"], ref["scales"], ref["gscale"], rows, cols, axis,
                             out_bf16=dtype == torch.bfloat16)
    p = torch.from_numpy(ref["packed"]).cuda()
    s = torch.from_numpy(ref["scales"]).cuda()
    g = torch.tensor([ref["gscale"]], dtype=torch.float32, device="cuda")
    out = nv.dequantize(p, s, g, rows, cols, axis, dtype)
    got = out.view(torch.int16 if dtype == torch.bfloat16 else torch.int32).cpu().numpy()
    np.testing.assert_array_equal(got, want.view(got.dtype))


@pytest.mark.parametrize("axis", [AXIS_COLS, AXIS_ROWS])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_dequantize_tiny_scales_and_ragged(axis, dtype):
    """Blocks spanning many decades near the bottom of the binary32 range, so
    decoded values include binary32 and bf16 subnormals; the row layout has a
    partial last chunk (37*80/16 = 185 blocks)."""
    banner(f"dequantize tiny axis={axis} {dtype}")
    rows, cols = (37, 80) if axis == AXIS_COLS else (80, 37)
    rng = np.random.default_rng(7)
    mag = 10.0 ** rng.uniform(-38, -33, (rows * cols) // 16)
    v = (rng.standard_normal(rows * cols) * np.repeat(mag, 16)).astype(np.float32)
    x = ((v.view(np.uint32) + 0x8000) >> 16).astype(np.uint16).reshape(rows, cols)
    ref = oracle.quantize(x, axis, F46, MSE)
    want = oracle.dequantize(ref["packed"], ref["scales"], ref["gscale"], rows, cols, axis,
                             out_bf16=dtype == torch.bfloat16)
    assert np.any((want.view(np.float32 if dtype == torch.float32 else np.uint16) != 0))
    p = torch.from_numpy(ref["packed"]).cuda()
    s = torch.from_numpy(ref["scales"]).cuda()
    g = torch.tensor([ref["gscale"]], dtype=torch.float32, device="cuda")
    out = nv.dequantize(p, s, g, rows, cols, axis, dtype)
    got = out.view(torch.int16 if dtype == torch.bfloat16 else torch.int32).cpu().numpy()
    np.testing.assert_array_equal(got, want.view(got.dtype))


@pytest.mark.parametrize("axis,cid", [(AXIS_ROWS, 5), (AXIS_COLS, 2)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_dequantize_full_size(axis, cid, dtype):
    """Dequantize the full column-blocked gradient workload (and a row-wise
    one) against the oracle's reconstruction, bit for bit."""
    cfg = testkit.WORKLOADS[cid]
    banner(f"dequantize full {cfg.rows}x{cfg.cols} axis={axis} {dtype}")
    x = testkit.make(cid)
    ref = oracle.quantize(x, axis, cfg.mode, cfg.rule, want_err=False)
    want = oracle.dequantize(ref["packed"], ref["scales"], ref["gscale"], cfg.rows, cfg.cols, axis,
                             out_bf16=dtype == torch.bfloat16)
    p = torch.from_numpy(ref["packed"]).cuda()
    s = torch.from_numpy(ref["scales"]).cuda()
    g = torch.tensor([ref["gscale"]], dtype=torch.float32, device="cuda")
    out = nv.dequantize(p, s, g, cfg.rows, cfg.cols, axis, dtype)
    got = out.view(torch.int16 if dtype == torch.bfloat16 else torch.int32).cpu().numpy()
    np.testing.assert_array_equal(got, want.view(got.dtype))


def test_round_trip_config1_through_gpu_outputs():
    banner("config 1 round trip")
    x = testkit.make(1)
    xd = to_device(x)
    r = nv.quantize(xd, AXIS_COLS, STD, MSE)
    out = nv.dequantize(r["packed"], r["scales"], r["gscale"], 256, 1024, AXIS_COLS)
    ref = oracle.quantize(x, AXIS_COLS, STD, MSE)
    want = oracle.dequantize(ref["packed"], ref["scales"], ref["gscale"], 256, 1024, AXIS_COLS)
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), want.view(np.uint32))


# ------------------------------------------------------------ delayed scaling ----

@pytest.mark.parametrize("axis,shape", [(AXIS_COLS, (512, 5120)), (AXIS_COLS, (37, 80)),
                                        (AXIS_ROWS, (1040, 72)), (AXIS_ROWS, (256, 130))])
@pytest.mark.parametrize("rule", [MSE, MAXE])
def test_delayed_scaling(axis, shape, rule):
    """Quantize with the previous tensor's scale while recording this
    tensor's amax: outputs equal the oracle's for that given g, the amax is
    exact, and the next call's g follows from it."""
    banner(f"delayed axis={axis} {shape} rule={rule}")
    x_prev = testkit.fill(shape, testkit.NORMAL, 2.0, 11 + shape[0])
    x = testkit.fill(shape, testkit.STUDENT_T3, 0.7, 13 + shape[1])
    g = nv.global_scale(nv.amax(to_device(x_prev)), F46)
    d = nv.quantize_delayed(to_device(x), g, axis, F46, rule, selmap=True, err_sum=True)
    torch.cuda.synchronize()
    g32 = np.float32(g.item())
    ref = oracle.quantize(x, axis, F46, rule, gscale=g32)
    np.testing.assert_array_equal(d["packed"].cpu().numpy().reshape(-1), ref["packed"])
    np.testing.assert_array_equal(d["scales"].cpu().numpy().reshape(-1), ref["scales"])
    np.testing.assert_array_equal(d["selmap"].cpu().numpy()[: ref["selmap"].size], ref["selmap"])
    assert d["err_sum"].item() == pytest.approx(ref["err_sum"], rel=1e-6)
    a = oracle.amax(x)
    assert np.float32(d["amax"].item()).view(np.uint32) == a.view(np.uint32)
    g_next = nv.global_scale(d["amax"], F46)
    assert np.float32(g_next.item()).view(np.uint32) == oracle.global_scale(a, F46).view(np.uint32)


def test_delayed_scaling_full_size_rows_sampled():
    banner("delayed 32768x5120")
    x = testkit.make(4)
    xd = to_device(x)
    g = torch.tensor([np.float32(0.75) * oracle.global_scale(oracle.amax(x), F46)],
                     dtype=torch.float32, device="cuda")  # a stale, smaller amax
    d = nv.quantize_delayed(xd, g, AXIS_COLS, F46, MSE)
    torch.cuda.synchronize()
    assert np.float32(d["amax"].item()).view(np.uint32) == oracle.amax(x).view(np.uint32)
    rng = np.random.default_rng(8)
    pick = np.unique(np.concatenate([[0, x.shape[0] - 1], rng.integers(0, x.shape[0], 30)]))
    ref = oracle.quantize(x[pick], AXIS_COLS, F46, MSE, gscale=np.float32(g.item()),
                          want_err=False)
    idx = torch.from_numpy(pick).cuda()
    np.testing.assert_array_equal(d["packed"][idx].cpu().numpy().reshape(-1), ref["packed"])
    np.testing.assert_array_equal(d["scales"][idx].cpu().numpy().reshape(-1), ref["scales"])


# ------------------------------------------------------------ dual layout ----

DUAL_SHAPES = [(16, 16), (48, 80), (272, 48), (1040, 80), (256, 144), (2048, 208)]


@pytest.mark.parametrize("rows,cols", DUAL_SHAPES)
@pytest.mark.parametrize("mode,rule", RULES)
def test_dual_layout_equals_single_layouts(rows, cols, mode, rule):
    """Both layouts from one read are bit-identical to the two single-layout
    calls with the same g, and to the oracle."""
    banner(f"dual {rows}x{cols} mode={mode} rule={rule}")
    x = testkit.fill((rows, cols), testkit.STUDENT_T3, 0.6, 3000 + rows + 7 * cols)
    xd = to_device(x)
    d = nv.quantize_dual(xd, mode, rule, selmap=True, err_sum=True)
    g = d["gscale"]
    for side, axis in (("rows", AXIS_COLS), ("cols", AXIS_ROWS)):
        s = nv.quantize(xd, axis, mode, rule, gscale=g.clone(), selmap=True, err_sum=True)
        for k in ("packed", "scales", "selmap"):
            assert torch.equal(d[side][k], s[k]), (side, k)
        assert d[side]["err_sum"].item() == pytest.approx(s["err_sum"].item(), rel=1e-12)
        ref = oracle.quantize(x, axis, mode, rule)
        assert np.float32(g.item()).view(np.uint32) == ref["gscale"].view(np.uint32)
        np.testing.assert_array_equal(d[side]["packed"].cpu().numpy().reshape(-1), ref["packed"])
        np.testing.assert_array_equal(d[side]["scales"].cpu().numpy().reshape(-1), ref["scales"])
        np.testing.assert_array_equal(d[side]["selmap"].cpu().numpy()[: ref["selmap"].size],
                                      ref["selmap"])
        assert d[side]["err_sum"].item() == pytest.approx(ref["err_sum"], rel=1e-6)


def test_dual_layout_full_size():
    banner("dual 8192x5120")
    x = testkit.make(5)
    xd = to_device(x)
    d = nv.quantize_dual(xd, F46, MAE)
    for side, axis in (("rows", AXIS_COLS), ("cols", AXIS_ROWS)):
        ref = oracle.quantize(x, axis, F46, MAE, want_err=False)
        np.testing.assert_array_equal(d[side]["packed"].cpu().numpy().reshape(-1), ref["packed"])
        np.testing.assert_array_equal(d[side]["scales"].cpu().numpy().reshape(-1), ref["scales"])
