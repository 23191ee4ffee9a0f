"""Device codec sweeps: the quantization kernels' own E2M1 and E4M3 encoders
and decoders, run on the GPU over every fp32 input of the ranges they see,
against the CPU reference.

* E2M1 encoder: every fp32 bit pattern in [0, 8] and in [-8, -0], and
  sampled ranges beyond 8 in magnitude (plus the infinities), against the
  oracle.
* E4M3 encoder: every fp32 bit pattern in [0, 464], against torch's
  float8_e4m3fn cast (pinned to the oracle by the CPU suite), plus a sampled
  comparison with the oracle itself and the saturation range.
* Decoders: all 16 E2M1 codes and all 127 finite E4M3 bytes, and the
  reciprocal table, against the oracle.
"""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_wave64_amd as nv
import oracle

pytestmark = pytest.mark.gpu

CHUNK = 1 << 27


def f32_bits(v):
    return int(np.float32(v).view(np.uint32))


def sweep(fn, first, count):
    out = torch.empty(count, dtype=torch.uint8, device="cuda")
    st = getattr(nv.lib(), fn)(first, count, out.data_ptr(), None)
    assert st == 0
    return out.cpu().numpy()


@pytest.mark.parametrize("sign", [0, 0x80000000])
def test_e2m1_encoder_every_pattern_in_plus_minus_8(sign):
    hi = f32_bits(8.0)
    for start in range(0, hi + 1, CHUNK):
        n = min(CHUNK, hi + 1 - start)
        print(f"\n[gpu-codecs] e2m1 bits {sign + start:#x}+{n}", flush=True)
        got = sweep("nvfp4v_e2m1_encode_sweep", sign + start, n)
        a = np.arange(start, start + n, dtype=np.uint32).view(np.float32)
        want = oracle.e2m1_index_array(a) | (8 if sign else 0)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (sign, a[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_e2m1_encoder_negative_and_large():
    rng = np.random.default_rng(12)
    for lo, hi in [(f32_bits(8.0), 0x7F800000), (0x80000000 + f32_bits(8.0), 0xFF800000)]:
        start = int(rng.integers(lo, hi - (1 << 22)))
        got = sweep("nvfp4v_e2m1_encode_sweep", start, 1 << 22)
        a = np.arange(start, start + (1 << 22), dtype=np.uint32).view(np.float32)
        want = oracle.e2m1_index_array(np.abs(a)) | (np.signbit(a).astype(np.uint8) << 3)
        np.testing.assert_array_equal(got, want)
    # infinities saturate like the oracle
    assert sweep("nvfp4v_e2m1_encode_sweep", 0x7F800000, 1)[0] == 7
    assert sweep("nvfp4v_e2m1_encode_sweep", 0xFF800000, 1)[0] == 15


def _torch_e4m3(s):
    return torch.from_numpy(s).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encoder_every_pattern_0_to_464():
    hi = f32_bits(464.0)
    rng = np.random.default_rng(0)
    for start in range(0, hi + 1, CHUNK):
        n = min(CHUNK, hi + 1 - start)
        print(f"\n[gpu-codecs] e4m3 bits {start:#x}+{n}", flush=True)
        got = sweep("nvfp4v_e4m3_encode_sweep", start, n)
        s = np.arange(start, start + n, dtype=np.uint32).view(np.float32)
        want = _torch_e4m3(s)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (s[bad[:5]], got[bad[:5]], want[bad[:5]])
        pick = rng.integers(0, n, 20000)
        np.testing.assert_array_equal(got[pick], oracle.e4m3_encode_array(s[pick]))


def test_e4m3_encoder_saturation_and_non_positive():
    start = f32_bits(464.0) + 1
    n = 0x7F800001 - start
    for first in range(start, start + n, CHUNK):
        cnt = min(CHUNK, start + n - first)
        got = sweep("nvfp4v_e4m3_encode_sweep", first, cnt)
        assert (got == 0x7E).all()
    got = sweep("nvfp4v_e4m3_encode_sweep", 0x80000000, 1 << 20)  # -0 and negatives
    assert (got == 0).all()
    got = sweep("nvfp4v_e4m3_encode_sweep", 0x7FC00000, 1 << 16)  # NaNs
    assert (got == 0).all()


@pytest.mark.parametrize("g", [1.0, 0.0390625, 3.0e-5, 7.5e30, 0.0, 2.0 ** -140])
def test_decode_and_scale_tables(g):
    """The kernels' E2M1 / E4M3 decoders and the per-scale multipliers
    d = dec(S) * g and r = min((1/g) * (1/dec(S)), FLT_MAX), against the
    oracle's block pipeline (blocks built so that each scale byte occurs)."""
    e2 = torch.empty(16, dtype=torch.float32, device="cuda")
    e4 = torch.empty(128, dtype=torch.float32, device="cuda")
    d = torch.empty(128, dtype=torch.float32, device="cuda")
    r = torch.empty(128, dtype=torch.float32, device="cuda")
    assert nv.lib().nvfp4v_decode_tables(float(np.float32(g)), e2.data_ptr(), e4.data_ptr(),
                                         d.data_ptr(), r.data_ptr(), None) == 0
    e2, e4, d, r = (t.cpu().numpy() for t in (e2, e4, d, r))
    want2 = np.array([oracle.e2m1_decode(c) for c in range(16)], np.float32)
    np.testing.assert_array_equal(e2.view(np.uint32), want2.view(np.uint32))
    want4 = np.array([oracle.e4m3_decode(S) for S in range(127)], np.float32)
    np.testing.assert_array_equal(e4[:127].view(np.uint32), want4.view(np.uint32))
    # The oracle's d and r for every scale byte: a block whose max is chosen
    # so that the max->6 candidate lands exactly on scale S.
    g32 = np.float32(g)
    for S in range(127):
        G = np.float32(1) / g32 if g32 != 0 else np.float32(np.inf)
        if not (0 < G <= np.finfo(np.float32).max):
            continue
        x = np.zeros(16, np.float32)
        x[0] = np.float32(want4[S]) * np.float32(6) * g32  # b = 6 * dec(S) * g
        q = oracle.quantize_block(x, g32, oracle.MODE_STD, oracle.RULE_MSE)
        if q.S[0] != S:
            continue  # rounding moved the block to a neighbouring scale
        assert np.float32(q.d[0]).view(np.uint32) == d[S].view(np.uint32), S
        assert np.float32(q.r[0]).view(np.uint32) == r[S].view(np.uint32), S
