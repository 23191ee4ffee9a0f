"""nvfp4_gemm_splitk_noalloc: the split-K W4A4 product with the per-range
sums in the library's fixed device scratch instead of a caller workspace
(for callers that cannot allocate).  Through the C ABI, its output must equal
nvfp4_gemm_splitk's with the same split count bit for bit (the same kernels,
a deterministic order), and lie within the header's bound of the oracle's
binary64 product -- on two calls in a row, the second smaller than the first
(so the scratch holds the larger call's sums when the smaller one starts),
then the first shape again.  Sizes past the scratch are refused before any
launch."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_wave64_amd as nv
import oracle

pytestmark = pytest.mark.gpu


def operand(seed, rows, K):
    rng = np.random.default_rng(seed)
    packed = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    scales = rng.integers(0x20, 0x50, (rows, K // 16), dtype=np.uint8)
    g = np.float32(0.5 + 0.25 * (seed % 3))
    dev = {"packed": torch.from_numpy(packed).cuda(), "scales": torch.from_numpy(scales).cuda(),
           "gscale": torch.tensor([float(g)], dtype=torch.float32, device="cuda")}
    return packed, scales, g, dev


def one_case(M, N, K, splits, seed, out_dtype):
    print(f"\n[no-alloc] {M}x{N}x{K}, {splits} splits, {out_dtype}", flush=True)
    pa, sa, ga, a = operand(seed, M, K)
    pb, sb, gb, b = operand(seed + 1, N, K)
    ref = torch.empty((M, N), dtype=out_dtype, device="cuda")
    ws = torch.empty(splits * M * N, dtype=torch.float32, device="cuda")
    nv.gemm(a, b, out_dtype, out=ref, splits=splits, workspace=ws)
    got = torch.full((M, N), float("nan"), dtype=out_dtype, device="cuda")
    nv.gemm_splitk_noalloc(a, b, splits, got)
    torch.cuda.synchronize()
    gi = got.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32).cpu().numpy()
    ri = ref.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32).cpu().numpy()
    np.testing.assert_array_equal(gi, ri)  # bit for bit the workspace entry point's
    want, wabs = oracle.gemm(pa, sa, ga, pb, sb, gb, M, N, K, want_abs=True)
    tol = (K + K // 16 + 2) * 2.0 ** -23 * wabs + 2.0 ** -126
    if out_dtype == torch.bfloat16:
        tol = tol + np.abs(want) * 2.0 ** -8
    err = np.abs(got.float().cpu().numpy().astype(np.float64) - want)
    assert np.all(err <= tol)


def test_two_calls_in_a_row_second_smaller():
    one_case(300, 520, 2048, 4, 11, torch.float32)   # 624,000 scratch floats
    one_case(70, 96, 640, 3, 21, torch.bfloat16)     # smaller, stale sums beyond it
    one_case(300, 520, 2048, 4, 31, torch.float32)   # the larger shape again, new operands


def test_largest_fitting_and_refused_sizes():
    # splits * M * N exactly at the limit (2^23) runs; one row more is refused.
    M, N, K, splits = 512, 4096, 1024, 4
    assert splits * M * N == nv.NOALLOC_SCRATCH_FLOATS
    one_case(M, N, K, splits, 41, torch.bfloat16)
    _, _, _, a = operand(51, M + 1, K)
    _, _, _, b = operand(52, N, K)
    out = torch.empty((M + 1, N), dtype=torch.float32, device="cuda")
    with pytest.raises(nv.NVFP4Error, match="NVFP4_ERR_SCRATCH"):
        nv.gemm_splitk_noalloc(a, b, splits, out)
