"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
binding and the oracle on the same host buffer, and compare."""
import numpy as np
import torch

import nvfp4_block_scaled_wave64_amd as nv
import oracle

GUARD = 256  # canary bytes before and after every output buffer
CANARY = 0xA5


def to_device(x_bf16):
    """uint16 host array -> contiguous bf16 device tensor (same bits)."""
    t = torch.from_numpy(np.ascontiguousarray(x_bf16).view(np.int16)).cuda()
    return t.view(torch.bfloat16)


class Guarded:
    """A device byte buffer with canary bands on both sides."""

    def __init__(self, nbytes, dtype=torch.uint8, align=256):
        self.nbytes = nbytes
        self.raw = torch.full((nbytes + 2 * GUARD,), CANARY, dtype=torch.uint8, device="cuda")
        self.view = self.raw[GUARD:GUARD + nbytes]
        if dtype != torch.uint8:
            self.view = self.view.view(dtype)

    def check(self):
        raw = self.raw.cpu().numpy()
        assert (raw[:GUARD] == CANARY).all(), "write before the buffer"
        assert (raw[GUARD + self.nbytes:] == CANARY).all(), "write past the buffer"


def gpu_quantize(x_bf16, block_axis, mode, rule, gscale=None, selmap=True, err=True,
                 stream=None):
    """Quantize through the C ABI with guarded outputs; returns host arrays."""
    rows, cols = x_bf16.shape
    n = rows * cols
    xd = to_device(x_bf16)
    bufs = {
        "packed": Guarded(n // 2),
        "scales": Guarded(n // 16),
        "gscale": Guarded(4, torch.float32),
    }
    nsel = (n // 16 + 7) // 8
    if selmap:
        bufs["selmap"] = Guarded(nsel)
    if err:
        bufs["err_sum"] = Guarded(8, torch.float64)
    g_arg = None
    if gscale is not None:
        bufs["gscale"].view.fill_(float(np.float32(gscale)))
        g_arg = bufs["gscale"].view
    out = {k: b.view for k, b in bufs.items()}
    nv.quantize(xd, block_axis, mode, rule, gscale=g_arg, selmap=selmap, err_sum=err, out=out,
                stream=stream)
    torch.cuda.synchronize()
    for b in bufs.values():
        b.check()
    res = {
        "packed": bufs["packed"].view.cpu().numpy(),
        "scales": bufs["scales"].view.cpu().numpy(),
        "gscale": np.float32(bufs["gscale"].view.cpu().numpy()[0]),
    }
    if selmap:
        res["selmap"] = bufs["selmap"].view.cpu().numpy()
    if err:
        res["err_sum"] = float(bufs["err_sum"].view.cpu().numpy()[0])
    return res


def assert_same(gpu, ref, what=""):
    """Bit-exact comparison of codes, scales, g and bitmap; err_sum within
    1e-6 relative (binary64 sums in different orders)."""
    assert gpu["gscale"].view(np.uint32) == np.float32(ref["gscale"]).view(np.uint32), what
    for key in ("scales", "packed", "selmap"):
        if key in gpu and ref.get(key) is not None:
            a, b = gpu[key], ref[key]
            bad = np.nonzero(a != b)[0]
            assert bad.size == 0, f"{what} {key}: {bad.size} mismatches, first at {bad[:8]}: " \
                                  f"gpu {a[bad[:8]]} oracle {b[bad[:8]]}"
    if "err_sum" in gpu and ref.get("err_sum") is not None:
        r = ref["err_sum"]
        if not (np.isfinite(r) and np.isfinite(gpu["err_sum"])):
            # Blocks whose squared error overflows binary32 make the sum +inf
            # on both sides; non-finite sums must agree exactly.
            assert gpu["err_sum"] == r, (what, gpu["err_sum"], r)
        else:
            assert abs(gpu["err_sum"] - r) <= 1e-6 * abs(r) + 1e-300, (what, gpu["err_sum"], r)


def check_against_oracle(x, block_axis, mode, rule, gscale=None, selmap=True, err=True, what=""):
    gpu = gpu_quantize(x, block_axis, mode, rule, gscale, selmap, err)
    ref = oracle.quantize(x, block_axis, mode, rule, gscale=gscale, want_selmap=selmap,
                          want_err=err)
    assert_same(gpu, ref, what)
    return gpu, ref
