"""Concurrency and graph capture through the C ABI.

* Calls on different streams share no state: two tensors quantized at the
  same time on two streams give the outputs of sequential calls.
* The whole quantize path (zeroing, amax, g, quantize) and the dequantizer
  launch kernels only (no memset nodes, no host synchronization), so they
  can be captured in a HIP graph: every replay, with new input copied into
  the captured buffer and eager work and synchronizations in between,
  must equal the eager result.
"""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_wave64_amd as nv
import oracle
import testkit
from tests._parity import to_device

pytestmark = pytest.mark.gpu
F46, MSE = nv.MODE_4OVER6, nv.RULE_MSE


def banner(msg):
    print(f"\n[gpu-streams] {msg}", flush=True)


def test_two_streams_concurrently():
    banner("two streams")
    xa = to_device(testkit.make(4, rows=4096))
    xb = to_device(testkit.make(5, rows=2048, cols=1024))
    ref_a = nv.quantize(xa, nv.AXIS_COLS, F46, MSE, selmap=True, err_sum=True)
    ref_b = nv.quantize(xb, nv.AXIS_ROWS, F46, nv.RULE_MAE, selmap=True, err_sum=True)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            a = nv.quantize(xa, nv.AXIS_COLS, F46, MSE, selmap=True, err_sum=True, stream=s1)
        with torch.cuda.stream(s2):
            b = nv.quantize(xb, nv.AXIS_ROWS, F46, nv.RULE_MAE, selmap=True, err_sum=True,
                            stream=s2)
        outs.append((a, b))
    torch.cuda.synchronize()
    for a, b in outs:
        for k in ("packed", "scales", "selmap", "gscale"):
            assert torch.equal(a[k], ref_a[k]), k
            assert torch.equal(b[k], ref_b[k]), k
        assert a["err_sum"].item() == pytest.approx(ref_a["err_sum"].item(), rel=1e-12)
        assert b["err_sum"].item() == pytest.approx(ref_b["err_sum"].item(), rel=1e-12)


@pytest.mark.parametrize("axis", [nv.AXIS_COLS, nv.AXIS_ROWS])
def test_graph_capture_and_replay(axis):
    banner(f"graph capture axis={axis}")
    rows, cols = 1024, 2048
    inputs = [testkit.fill((rows, cols), testkit.STUDENT_T3, s, 100 + i)
              for i, s in enumerate((0.5, 3.0, 0.01, 40.0))]
    static_x = to_device(inputs[0])
    pshape, sshape, nsel = nv.output_shapes(rows, cols, axis)
    out = {"packed": torch.empty(pshape, dtype=torch.uint8, device="cuda"),
           "scales": torch.empty(sshape, dtype=torch.uint8, device="cuda"),
           "selmap": torch.empty(nsel, dtype=torch.uint8, device="cuda"),
           "err_sum": torch.empty(1, dtype=torch.float64, device="cuda"),
           "gscale": torch.empty(1, dtype=torch.float32, device="cuda")}
    xhat = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")

    def path():
        nv.quantize(static_x, axis, F46, MSE, selmap=True, err_sum=True, out=out)
        nv.dequantize(out["packed"], out["scales"], out["gscale"], rows, cols, axis,
                      torch.bfloat16, out=xhat)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        path()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        path()
    torch.cuda.synchronize()
    for i, x in enumerate(inputs + inputs[:1]):
        static_x.copy_(to_device(x))
        graph.replay()
        torch.cuda.synchronize()
        got = {k: v.clone() for k, v in out.items()}
        got_xhat = xhat.clone()
        # eager work between replays
        eager = nv.quantize(to_device(x), axis, F46, MSE, selmap=True, err_sum=True)
        eager_xhat = nv.dequantize(eager["packed"], eager["scales"], eager["gscale"], rows, cols,
                                   axis, torch.bfloat16)
        torch.cuda.synchronize()
        for k in ("packed", "scales", "selmap", "gscale"):
            assert torch.equal(got[k], eager[k]), (i, k)
        assert got["err_sum"].item() == pytest.approx(eager["err_sum"].item(), rel=1e-12)
        assert torch.equal(got_xhat.view(torch.int16), eager_xhat.view(torch.int16)), i
        ref = oracle.quantize(x, axis, F46, MSE, want_err=False)
        np.testing.assert_array_equal(got["scales"].cpu().numpy().reshape(-1), ref["scales"])


def test_outlier_channels_and_w4a4_product_in_a_graph():
    """The augmented layer (residual quantize of the activations, then the
    W4A4 product with the duplicated weight) captured once and replayed on
    new activations; each replay equals the eager calls bit for bit."""
    banner("graph capture: residual quantize + W4A4 product")
    rows, cols, n_out, nres = 512, 1024, 384, 64
    w = to_device(testkit.fill((n_out, cols), testkit.NORMAL, 0.02, 7))
    calib = to_device(testkit.fill((rows, cols), testkit.STUDENT_T3, 0.5, 8))
    _, perm = nv.channel_order(calib)
    qw = nv.quantize_residual(w, perm, nres, F46, MSE, duplicate=True)
    inputs = [testkit.fill((rows, cols), testkit.STUDENT_T3, s, 200 + i)
              for i, s in enumerate((0.5, 4.0, 0.02))]
    static_x = to_device(inputs[0])
    qa = nv.quantize_residual(static_x, perm, nres, F46, MSE)
    y = torch.empty((rows, n_out), dtype=torch.bfloat16, device="cuda")

    def layer():
        nv.quantize_residual(static_x, perm, nres, F46, MSE, out=qa)
        nv.gemm(qa, qw, torch.bfloat16, out=y)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer()
    torch.cuda.synchronize()
    for i, x in enumerate(inputs + inputs[:1]):
        static_x.copy_(to_device(x))
        graph.replay()
        torch.cuda.synchronize()
        got = y.clone()
        ea = nv.quantize_residual(to_device(x), perm, nres, F46, MSE)
        ey = nv.gemm(ea, qw, torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(qa["packed"], ea["packed"]) and torch.equal(qa["scales"], ea["scales"]), i
        assert torch.equal(got.view(torch.int16), ey.view(torch.int16)), i
