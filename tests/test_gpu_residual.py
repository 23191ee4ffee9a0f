"""GPU parity of the outlier-channel path ("ARCQuant" summary, gist.science
2601.07475, "Methodology"): the per-channel maxima, the channel order and the
two-stage (primary + residual) quantization through the C ABI, bit-exact
against the oracle on the same seeded inputs.

Shapes span the kernels' launch regimes: one row per wave (cols <= 8192,
each row-buffer size class, including rows shorter than a wave's 64
blocks), rows shared by a 1024-thread workgroup (wider rows, one to several
rows per step with a ragged last step, up to the 32768-channel limit),
column tiles with a partial last tile, and the 32768 x 5120 prefill
activations at full size."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_wave64_amd as nv
import oracle
import testkit
from tests._parity import Guarded, to_device

pytestmark = pytest.mark.gpu

STD, F46 = nv.MODE_STD, nv.MODE_4OVER6
MSE, MAE, MAXE = nv.RULE_MSE, nv.RULE_MAE, nv.RULE_MAX
RULES = [(STD, MSE), (F46, MSE), (F46, MAE), (F46, MAXE)]


def banner(msg):
    print(f"\n[gpu-residual] {msg}", flush=True)


def outlier_tensor(seed, rows, cols, n_out=8, factor=50.0):
    x = testkit.fill((rows, cols), testkit.STUDENT_T3, 0.5, seed)
    if n_out:
        testkit.scale_columns(x, testkit.sample(seed + 1, cols, min(n_out, cols)), factor)
    return x


def gpu_channel_order(x, absmax=None, accumulate=False):
    rows, cols = x.shape
    a = Guarded(cols * 4, torch.float32)
    p = Guarded(cols * 4, torch.int32)
    if absmax is not None:
        a.view.copy_(torch.from_numpy(absmax))
    nv.channel_order(to_device(x), absmax=a.view, accumulate=accumulate, perm=p.view)
    torch.cuda.synchronize()
    a.check()
    p.check()
    return a.view.cpu().numpy(), p.view.cpu().numpy()


def gpu_residual(x, perm, nres, mode, rule, gscale=None):
    rows, cols = x.shape
    width = cols + nres
    bufs = {"packed": Guarded(rows * width // 2), "scales": Guarded(rows * width // 16),
            "gscale": Guarded(4, torch.float32)}
    g_arg = None
    if gscale is not None:
        bufs["gscale"].view.fill_(float(np.float32(gscale)))
        g_arg = bufs["gscale"].view
    out = {k: b.view for k, b in bufs.items()}
    pd = torch.from_numpy(np.ascontiguousarray(perm, np.int32)).cuda()
    nv.quantize_residual(to_device(x), pd, nres, mode, rule, gscale=g_arg, out=out)
    torch.cuda.synchronize()
    for b in bufs.values():
        b.check()
    return {"packed": bufs["packed"].view.cpu().numpy().reshape(rows, width // 2),
            "scales": bufs["scales"].view.cpu().numpy().reshape(rows, width // 16),
            "gscale": np.float32(bufs["gscale"].view.cpu().numpy()[0])}


def assert_residual_same(got, ref, what):
    assert got["gscale"].view(np.uint32) == np.float32(ref["gscale"]).view(np.uint32), what
    for key in ("scales", "packed"):
        a, b = got[key], ref[key]
        bad = np.argwhere(a != b)
        assert bad.size == 0, f"{what}: {key} differs at {bad[:5].tolist()} ({len(bad)} total)"


# ------------------------------------------------------- channel order ----

ORDER_SHAPES = [(1, 16), (7, 48), (33, 1040), (1000, 80), (129, 5120), (64, 8208), (9, 32768)]


@pytest.mark.parametrize("rows,cols", ORDER_SHAPES)
def test_channel_order_matches_oracle(rows, cols):
    banner(f"channel order {rows}x{cols}")
    x = outlier_tensor(1000 + cols, rows, cols)
    a, p = gpu_channel_order(x)
    a_ref = oracle.channel_absmax(x)
    np.testing.assert_array_equal(a.view(np.uint32), a_ref.view(np.uint32))
    np.testing.assert_array_equal(p, oracle.channel_order(a_ref))


def test_channel_order_ties_and_zero_columns():
    """Equal maxima keep increasing channel order; all-zero and -0 columns
    rank last with maximum +0."""
    banner("channel order ties")
    rows, cols = 40, 512
    rng = np.random.default_rng(7)
    grid = np.array([0.5, 1.0, 1.5, 2.0], np.float32)
    xf = grid[rng.integers(0, 4, (rows, cols))] * rng.choice([-1, 1], (rows, cols))
    x = (xf.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    x[:, 3] = 0
    x[:, 100] = 0x8000
    a, p = gpu_channel_order(x)
    a_ref = oracle.channel_absmax(x)
    np.testing.assert_array_equal(a.view(np.uint32), a_ref.view(np.uint32))
    np.testing.assert_array_equal(p, oracle.channel_order(a_ref))
    assert a[3] == 0 and a[100] == 0 and not np.signbit(a[100])


def test_channel_order_accumulates_over_batches():
    """The running maximum over calibration batches: the order of two
    batches folded together equals the order of their concatenation."""
    banner("channel order accumulate")
    x1 = outlier_tensor(11, 300, 2048, n_out=4)
    x2 = outlier_tensor(12, 200, 2048, n_out=4)
    a1, _ = gpu_channel_order(x1)
    a, p = gpu_channel_order(x2, absmax=a1, accumulate=True)
    a_ref = oracle.channel_absmax(np.concatenate([x1, x2]))
    np.testing.assert_array_equal(a.view(np.uint32), a_ref.view(np.uint32))
    np.testing.assert_array_equal(p, oracle.channel_order(a_ref))


# -------------------------------------------------- residual quantize ----

RES_SHAPES = [
    # (rows, cols, nres): one row per wave for cols <= 8192 (every row-buffer
    # size class, fewer rows than waves), workgroup-shared rows above (one,
    # two and three rows per step, ragged last step), nres = 0 and nres = cols
    (1, 16, 16), (5, 48, 16), (37, 64, 0), (1000, 80, 32), (129, 1040, 112), (33, 5120, 256),
    (16, 8192, 512), (20, 8208, 1024), (3, 32768, 2048), (7, 256, 256), (37, 12288, 512),
    (300, 16384, 1024), (500, 4112, 64), (9, 4096, 128), (11, 5136, 48),
]


@pytest.mark.parametrize("rows,cols,nres", RES_SHAPES)
@pytest.mark.parametrize("mode,rule", RULES)
def test_quantize_residual_matches_oracle(rows, cols, nres, mode, rule):
    banner(f"residual {rows}x{cols} nres={nres} mode={mode} rule={rule}")
    x = outlier_tensor(2000 + cols + nres, rows, cols)
    perm = oracle.channel_order(oracle.channel_absmax(x))
    got = gpu_residual(x, perm, nres, mode, rule)
    ref = oracle.quantize_residual(x, perm, nres, mode, rule)
    assert_residual_same(got, ref, f"{rows}x{cols} nres={nres}")


def test_quantize_residual_given_scale_and_any_index_vector():
    """A given tensor scale, and an in-range index vector that is not a
    permutation (repeated and missing channels): gathered as given.
    (Entries out of range poison the output: see below.)"""
    banner("residual given scale, general index vector")
    rows, cols, nres = 50, 640, 64
    x = outlier_tensor(31, rows, cols)
    rng = np.random.default_rng(9)
    idx = rng.integers(0, cols, cols).astype(np.int32)
    idx[:5] = [0, 0, cols - 1, cols - 1, 3]
    g = np.float32(0.0123)
    got = gpu_residual(x, idx, nres, F46, MSE, gscale=g)
    ref = oracle.quantize_residual(x, idx, nres, F46, MSE, gscale=g)
    assert_residual_same(got, ref, "index vector")


def test_quantize_residual_all_zero_tensor():
    banner("residual zero tensor")
    x = np.zeros((24, 128), np.uint16)
    x[5, :] = 0x8000
    perm = np.arange(128, dtype=np.int32)
    got = gpu_residual(x, perm, 128, F46, MSE)
    ref = oracle.quantize_residual(x, perm, 128, F46, MSE)
    assert_residual_same(got, ref, "zeros")


def test_quantize_residual_full_size_prefill():
    """32768 x 5120 prefill activations (the Student-t recipe with 8 outlier
    channels x100), order from the GPU, 256 residual channels: the whole
    order and sampled rows of the outputs against the oracle."""
    banner("residual 32768x5120 full size")
    x = testkit.make(4)
    rows, cols, nres = 32768, 5120, 256
    a, p = gpu_channel_order(x)
    a_ref = oracle.channel_absmax(x)
    np.testing.assert_array_equal(a.view(np.uint32), a_ref.view(np.uint32))
    perm = oracle.channel_order(a_ref)
    np.testing.assert_array_equal(p, perm)
    got = gpu_residual(x, perm, nres, F46, MSE)
    g_ref = oracle.global_scale(oracle.amax(x), F46)
    rng = np.random.default_rng(5)
    pick = np.unique(np.concatenate([[0, 1, rows - 1], rng.integers(0, rows, 61)]))
    ref = oracle.quantize_residual(x[pick], perm, nres, F46, MSE, gscale=g_ref)
    assert got["gscale"].view(np.uint32) == g_ref.view(np.uint32)
    sub = {"packed": got["packed"][pick], "scales": got["scales"][pick], "gscale": got["gscale"]}
    assert_residual_same(sub, ref, "full size sampled rows")


# ------------------------------------------ RMSNorm + residual, fused ----

def gpu_rms_residual(x, w, eps, perm, nres, mode, rule, gscale=None, amax=False):
    rows, cols = x.shape
    width = cols + nres
    bufs = {"packed": Guarded(rows * width // 2), "scales": Guarded(rows * width // 16),
            "gscale": Guarded(4, torch.float32)}
    if amax:
        bufs["amax"] = Guarded(4, torch.float32)
    g_arg = None
    if gscale is not None:
        bufs["gscale"].view.fill_(float(np.float32(gscale)))
        g_arg = bufs["gscale"].view
    out = {k: b.view for k, b in bufs.items()}
    pd = torch.from_numpy(np.ascontiguousarray(perm, np.int32)).cuda()
    wd = None if w is None else to_device(w)
    nv.rmsnorm_quantize_residual(to_device(x), pd, nres, weight=wd, eps=eps, mode=mode, rule=rule,
                                 gscale=g_arg, amax=amax, out=out)
    torch.cuda.synchronize()
    for b in bufs.values():
        b.check()
    res = {"packed": bufs["packed"].view.cpu().numpy().reshape(rows, width // 2),
           "scales": bufs["scales"].view.cpu().numpy().reshape(rows, width // 16),
           "gscale": np.float32(bufs["gscale"].view.cpu().numpy()[0])}
    if amax:
        res["amax"] = np.float32(bufs["amax"].view.cpu().numpy()[0])
    return res


RMS_SHAPES = [
    # (rows, cols, nres): every row-buffer size class of the fused kernel,
    # fewer rows than waves, ragged row counts, nres = 0 and nres = cols;
    # past 8192 channels the workgroup-shared kernel with 3, 2 and 1 rows
    # per step, a partial last step, and its padded sum-of-squares tree
    # (8208 and 10240 channels: 1026 and 1280 chunks in a 2048-leaf tree)
    (1, 16, 16), (7, 48, 0), (100, 1040, 64), (33, 2048, 256), (65, 2064, 128), (40, 4096, 512),
    (11, 4112, 32), (19, 5120, 256), (5, 5136, 16), (25, 6144, 96), (13, 6160, 1024),
    (9, 8192, 8192), (6, 8208, 64), (4, 10240, 10240), (7, 12288, 512), (5, 16384, 1024),
    (33, 16384, 0), (3, 24576, 256),
]


@pytest.mark.parametrize("rows,cols,nres", RMS_SHAPES)
@pytest.mark.parametrize("weighted", [False, True])
def test_rmsnorm_residual_matches_oracle(rows, cols, nres, weighted):
    banner(f"rmsnorm+residual {rows}x{cols} nres={nres} weighted={weighted}")
    x = outlier_tensor(3000 + cols + nres, rows, cols)
    w = testkit.fill((cols,), testkit.NORMAL, 1.0, 77 + cols) if weighted else None
    eps = 1e-6
    y = oracle.rmsnorm(x, w, eps)
    perm = oracle.channel_order(oracle.channel_absmax(y))
    got = gpu_rms_residual(x, w, eps, perm, nres, F46, MSE, amax=True)
    ref = oracle.quantize_residual(y, perm, nres, F46, MSE)
    assert_residual_same(got, ref, f"{rows}x{cols}")
    assert got["amax"].view(np.uint32) == oracle.amax(y).view(np.uint32)


@pytest.mark.parametrize("mode,rule", RULES)
@pytest.mark.parametrize("rows,cols,nres", [(64, 3072, 192), (10, 16384, 384)])
def test_rmsnorm_residual_rules_and_given_scale(mode, rule, rows, cols, nres):
    banner(f"rmsnorm+residual rules mode={mode} rule={rule} {rows}x{cols}")
    x = outlier_tensor(41, rows, cols)
    w = testkit.fill((cols,), testkit.NORMAL, 0.5, 42)
    for eps in (0.0, 1e-2):
        y = oracle.rmsnorm(x, w, eps)
        perm = oracle.channel_order(oracle.channel_absmax(y))
        g = np.float32(0.0071)
        got = gpu_rms_residual(x, w, eps, perm, nres, mode, rule, gscale=g)
        ref = oracle.quantize_residual(y, perm, nres, mode, rule, gscale=g)
        assert_residual_same(got, ref, f"eps={eps}")


def test_rmsnorm_residual_zero_rows_and_large_values():
    """All-zero rows (y = 0 with eps > 0) and rows scaled near the bf16 top,
    whose squares stay finite in binary32."""
    banner("rmsnorm+residual zero rows, large values")
    rows, cols, nres = 12, 256, 32
    x = outlier_tensor(51, rows, cols)
    x[3] = 0
    x[7] = 0x8000
    xf = testkit.bf16_to_f32(x[5]) * np.float32(2.0 ** 40)
    x[5] = (xf.view(np.uint32) >> 16).astype(np.uint16)
    y = oracle.rmsnorm(x, None, 1e-5)
    perm = oracle.channel_order(oracle.channel_absmax(y))
    got = gpu_rms_residual(x, None, 1e-5, perm, nres, F46, MAE)
    ref = oracle.quantize_residual(y, perm, nres, F46, MAE)
    assert_residual_same(got, ref, "zeros/large")


def test_rmsnorm_residual_full_size_prefill():
    """32768 x 5120 prefill activations through the fused path (weight,
    256 residual channels, g from the first pass), sampled rows against the
    oracle."""
    banner("rmsnorm+residual 32768x5120 full size")
    x = testkit.make(4)
    rows, cols, nres = 32768, 5120, 256
    w = testkit.fill((cols,), testkit.NORMAL, 1.0, 99)
    eps = 1e-6
    y = oracle.rmsnorm(x, w, eps)
    perm = oracle.channel_order(oracle.channel_absmax(y))
    got = gpu_rms_residual(x, w, eps, perm, nres, F46, MSE, amax=True)
    g_ref = oracle.global_scale(oracle.amax(y), F46)
    assert got["gscale"].view(np.uint32) == g_ref.view(np.uint32)
    assert got["amax"].view(np.uint32) == oracle.amax(y).view(np.uint32)
    rng = np.random.default_rng(6)
    pick = np.unique(np.concatenate([[0, 1, rows - 1], rng.integers(0, rows, 61)]))
    ref = oracle.quantize_residual(y[pick], perm, nres, F46, MSE, gscale=g_ref)
    sub = {"packed": got["packed"][pick], "scales": got["scales"][pick], "gscale": got["gscale"]}
    assert_residual_same(sub, ref, "full size sampled rows")


# ------------------------------------------------- invalid channel orders ----

@pytest.mark.parametrize("cols", [16, 80, 5120, 8208, 32768])
def test_check_order_counts_what_breaks_a_permutation(cols):
    """nvfp4_check_order: 0 for permutations; out-of-range entries and
    repeats counted as cols - (distinct in-range values)."""
    banner(f"check_order cols={cols}")
    rng = np.random.default_rng(cols)
    perm = rng.permutation(cols).astype(np.int32)
    cases = [(perm, 0), (perm[::-1].copy(), 0)]
    p1 = perm.copy(); p1[cols // 2] = cols; cases.append((p1, 1))
    p2 = perm.copy(); p2[0] = -1; p2[-1] = 1 << 30; cases.append((p2, 2))
    if cols > 1:
        p3 = perm.copy(); p3[1] = p3[0]; cases.append((p3, 1))
    cases.append((np.zeros(cols, np.int32), cols - 1))
    for p, want in cases:
        bad = nv.check_order(torch.from_numpy(p).cuda())
        torch.cuda.synchronize()
        assert int(bad.cpu().numpy()[0]) == want


@pytest.mark.parametrize("rows,cols,nres,rms", [
    (37, 80, 16, False), (300, 5120, 256, False), (20, 9216, 512, False),  # both kernel shapes
    (37, 80, 16, True), (300, 5120, 256, True),  # fused RMSNorm, one row per wave
    (9, 16384, 512, True),  # fused RMSNorm, rows shared by a workgroup
])
def test_out_of_range_order_poisons_the_output(rows, cols, nres, rms):
    """An order entry outside [0, cols) makes nvfp4_quantize_residual (and
    the fused RMSNorm call) write 0x7F (E4M3 NaN) into every scale byte and
    0 into every code; dequantizing gives NaN everywhere, and so does a
    W4A4 product over it.  The same call with a valid order is checked
    against the oracle first, so the outputs are known to be overwritten."""
    banner(f"poisoned output {rows}x{cols}, nres={nres}, rms={rms}")
    x = outlier_tensor(7 + cols, rows, cols)
    xd = to_device(x)
    perm = oracle.channel_order(oracle.channel_absmax(x))
    width = cols + nres
    out = {"packed": torch.empty(rows * width // 2, dtype=torch.uint8, device="cuda"),
           "scales": torch.empty(rows * width // 16, dtype=torch.uint8, device="cuda"),
           "gscale": torch.empty(1, dtype=torch.float32, device="cuda")}

    def call(p):
        pd = torch.from_numpy(p.astype(np.int32)).cuda()
        if rms:
            nv.rmsnorm_quantize_residual(xd, pd, nres, out=out)
        else:
            nv.quantize_residual(xd, pd, nres, out=out)
        torch.cuda.synchronize()
        return out["packed"].cpu().numpy(), out["scales"].cpu().numpy()

    good_p, good_s = call(perm)
    if not rms:
        ref = oracle.quantize_residual(x, perm, nres, F46, MSE)
        np.testing.assert_array_equal(good_s, ref["scales"].reshape(-1))
        np.testing.assert_array_equal(good_p, ref["packed"].reshape(-1))
    assert (good_s != 0x7F).all()
    for bad_value in (cols, -5):
        p = perm.copy()
        p[cols // 3] = bad_value
        assert int(nv.check_order(torch.from_numpy(p.astype(np.int32)).cuda()).cpu()[0]) == 1
        pk, sc = call(p)
        assert (sc == 0x7F).all(), "every scale byte must carry the NaN code"
        assert (pk == 0).all()
        deq = nv.dequantize(out["packed"], out["scales"], out["gscale"], rows, width,
                            nv.AXIS_COLS)
        assert torch.isnan(deq).all().item()
    w = testkit.fill((24, width), testkit.NORMAL, 0.02, 3)
    qw = nv.quantize(to_device(w), nv.AXIS_COLS, F46, MSE)
    a = {"packed": out["packed"].view(rows, width // 2), "scales": out["scales"].view(rows, width // 16),
         "gscale": out["gscale"]}
    b = {"packed": qw["packed"].view(24, width // 2), "scales": qw["scales"].view(24, width // 16),
         "gscale": qw["gscale"]}
    assert torch.isnan(nv.gemm(a, b)).all().item()


# ------------------------------------------- random finite bit patterns ----

def random_finite_patterns(shape, e_lo, e_hi, seed):
    """bf16 patterns with random sign and mantissa and an exponent field
    uniform in [e_lo, e_hi] (never 255: infinity and NaN are outside the
    contract)."""
    rng = np.random.default_rng(seed)
    sign = rng.integers(0, 2, shape, dtype=np.uint16) << 15
    exp = rng.integers(e_lo, e_hi + 1, shape, dtype=np.uint16) << 7
    man = rng.integers(0, 128, shape, dtype=np.uint16)
    return (sign | exp | man).astype(np.uint16)


@pytest.mark.parametrize("e_lo,e_hi", [(0, 24), (112, 142), (224, 254)])
@pytest.mark.parametrize("rows,cols,nres", [(37, 1040, 112), (19, 5120, 256), (9, 4096, 128),
                                            (5, 12288, 512)])
def test_quantize_residual_random_bit_patterns(e_lo, e_hi, rows, cols, nres):
    """Random finite patterns in one exponent window (subnormal-heavy, thirty
    binades around 1, the top of the range) through both stages: the
    lane-pair pass, the stash and the workgroup kernel, bit-exact."""
    banner(f"residual random patterns e=[{e_lo},{e_hi}] {rows}x{cols} nres={nres}")
    x = random_finite_patterns((rows, cols), e_lo, e_hi, 700 + e_lo + cols)
    perm = oracle.channel_order(oracle.channel_absmax(x))
    for mode, rule in ((F46, MSE), (F46, MAXE)):
        got = gpu_residual(x, perm, nres, mode, rule)
        ref = oracle.quantize_residual(x, perm, nres, mode, rule)
        assert_residual_same(got, ref, f"patterns e>={e_lo} {rows}x{cols} rule={rule}")


@pytest.mark.parametrize("e_lo,e_hi", [(0, 24), (112, 142), (224, 254)])
@pytest.mark.parametrize("cols", [5120, 16384])
def test_rmsnorm_residual_random_bit_patterns(e_lo, e_hi, cols):
    """The fused RMSNorm path on random finite patterns (squares that
    underflow, and sums of squares that overflow to +inf), with the first
    pass forming g: bit-exact, and the same max |y|."""
    banner(f"rmsnorm+residual random patterns e=[{e_lo},{e_hi}]")
    rows, nres = 23, 256
    x = random_finite_patterns((rows, cols), e_lo, e_hi, 800 + e_lo + cols)
    w = testkit.fill((cols,), testkit.NORMAL, 1.0, 81)
    eps = 1e-6
    y = oracle.rmsnorm(x, w, eps)
    perm = oracle.channel_order(oracle.channel_absmax(y))
    got = gpu_rms_residual(x, w, eps, perm, nres, F46, MSE, amax=True)
    ref = oracle.quantize_residual(y, perm, nres, F46, MSE)
    assert_residual_same(got, ref, f"patterns e>={e_lo}")
    assert got["amax"].view(np.uint32) == oracle.amax(y).view(np.uint32)


# ------------------------------------------ residual second-stage modes ----

STASH_SHAPES = [
    # (rows, cols, nres): residual blocks per row nrb = nres / 16 and rows per
    # wave chosen to cover every second-stage mode of the one-row-per-wave
    # kernel, with ragged per-wave row counts and several rows per wave:
    # the lane-pair pass after each row (nrb <= 32 at 4, 10 and 12 vectors
    # per lane: nrb = 2, 16, 17, 32), the 32-block stash of the kernels at 8
    # and 16 vectors per lane (passes over 2 and 4 rows, full and partial
    # batches), the 64-block stash (nrb = 48) and no stash (nrb = 80).
    (70001, 80, 32), (9221, 80, 32), (15367, 5120, 256), (7000, 1040, 272), (6000, 512, 512),
    (20000, 3072, 256), (9000, 8192, 128), (5000, 2048, 768), (4000, 2048, 1280),
]


@pytest.mark.parametrize("rows,cols,nres", STASH_SHAPES)
@pytest.mark.parametrize("mode,rule", [(F46, MSE), (F46, MAE)])
def test_quantize_residual_second_stage_modes(rows, cols, nres, mode, rule):
    banner(f"residual second-stage modes {rows}x{cols} nres={nres} rule={rule}")
    x = outlier_tensor(5000 + cols + nres, rows, cols)
    perm = oracle.channel_order(oracle.channel_absmax(x))
    got = gpu_residual(x, perm, nres, mode, rule)
    ref = oracle.quantize_residual(x, perm, nres, mode, rule)
    assert_residual_same(got, ref, f"stash {rows}x{cols} nres={nres}")
