"""The measurement entry points on the GPU: the timed quantize variant gives
the same outputs as the plain call and records its events on the quantize
kernels, and the access-pattern probes write exactly the bytes they
document (a check of their lane mapping, gathers and store offsets,
computed here on the host from the input)."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_wave64_amd as nv
import testkit
from tests._parity import to_device

pytestmark = pytest.mark.gpu


def banner(msg):
    print(f"\n[gpu-measure] {msg}", flush=True)


@pytest.mark.parametrize("axis,shape", [(nv.AXIS_COLS, (512, 5120)), (nv.AXIS_COLS, (37, 80)),
                                        (nv.AXIS_ROWS, (1024, 200))])
@pytest.mark.parametrize("given", [False, True])
def test_timed_variant_matches_plain_call(axis, shape, given):
    banner(f"timed axis={axis} shape={shape} given={given}")
    x = testkit.fill(shape, testkit.STUDENT_T3, 0.5, 77 + shape[0])
    xd = to_device(x)
    kw = dict(selmap=True, err_sum=True)
    a = nv.quantize(xd, axis, nv.MODE_4OVER6, nv.RULE_MSE, **kw)
    g = a["gscale"].clone() if given else None
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    b = nv.quantize(xd, axis, nv.MODE_4OVER6, nv.RULE_MSE, gscale=g, events=ev, **kw)
    torch.cuda.synchronize()
    for k in ("packed", "scales", "selmap", "gscale"):
        assert torch.equal(a[k], b[k]), k
    assert a["err_sum"].item() == pytest.approx(b["err_sum"].item(), rel=1e-12)
    ms = ev[0].elapsed_time(ev[1])
    assert 0.0 < ms < 1000.0


def test_timed_events_cover_only_the_quantize_kernel():
    """With the amax pass in the call, the bracketed time stays at the
    quantize kernel's: well below the whole call's time."""
    banner("timed bracket")
    x = testkit.make(4, rows=4096)
    xd = to_device(x)
    out = nv.quantize(xd, nv.AXIS_COLS, nv.MODE_4OVER6, nv.RULE_MSE, selmap=True, err_sum=True)
    inner = []
    for _ in range(5):
        ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        outer = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        outer[0].record()
        nv.quantize(xd, nv.AXIS_COLS, nv.MODE_4OVER6, nv.RULE_MSE, selmap=True, err_sum=True,
                    out=out, events=ev)
        outer[1].record()
        torch.cuda.synchronize()
        inner.append((ev[0].elapsed_time(ev[1]), outer[0].elapsed_time(outer[1])))
    for t_in, t_out in inner[1:]:
        assert 0.0 < t_in < t_out


@pytest.mark.parametrize("nblocks", [1, 63, 64, 1000, 64 * 4096 + 17])
def test_stream_pattern_bytes(nblocks):
    banner(f"stream pattern nblocks={nblocks}")
    x = testkit.fill((nblocks * 16,), testkit.NORMAL, 1.0, nblocks)
    xd = to_device(x)
    packed = torch.empty(nblocks * 8, dtype=torch.uint8, device="cuda")
    scales = torch.empty(nblocks, dtype=torch.uint8, device="cuda")
    nv.stream_pattern(xd, packed, scales)
    words = x.view(np.uint32).reshape(nblocks, 8)
    f = np.bitwise_xor.reduce(words[:, :4], axis=1)
    h = np.bitwise_xor.reduce(words[:, 4:], axis=1)
    want_packed = np.stack([f, h], axis=1).astype("<u4").view(np.uint8).reshape(-1)
    want_scales = ((f ^ h) & 0xFF).astype(np.uint8)
    np.testing.assert_array_equal(packed.cpu().numpy(), want_packed)
    np.testing.assert_array_equal(scales.cpu().numpy(), want_scales)


