"""Pins of the oracle's number formats against facts fixed outside the oracle.

* E2M1 magnitudes and step sizes: "Technical summary: Four Over Six (4/6)",
  "Problem statement" (steps 0.5 on [0,2], 1 on [2,4], 2 on [4,6]).
* E4M3 block scales and bf16 inputs: checked against torch's own
  float8_e4m3fn / bfloat16 casts (an independent implementation).
* E2M1 encoding: checked against the closed-form table of round-to-nearest-
  even decision points (a different formulation from the oracle's nearest-
  neighbour search), exhaustively over every fp32 pattern in [0, 8].
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

E2M1_GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def f32_bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def from_bits(u):
    return np.asarray(u, np.uint32).view(np.float32)


# ---------------------------------------------------------------- bf16 ----

def test_bf16_widening_all_patterns():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).float().numpy()
    got = np.array([oracle.bf16_to_f32(v) for v in h[::1]], np.float32)
    same = (got.view(np.uint32) == want.view(np.uint32)) | (np.isnan(got) & np.isnan(want))
    assert same.all()


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(7)
    u = rng.integers(0, 2**32, size=20000, dtype=np.uint64).astype(np.uint32)
    # ties and near-ties of the 16 dropped bits
    ties = (rng.integers(0, 2**16, size=4000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    u = np.concatenate([u, ties, ties + 1, ties - 1])
    f = from_bits(u)
    f = f[np.isfinite(f)]
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f32_to_bf16(v) for v in f], np.uint16)
    assert (got == want).all()


# ---------------------------------------------------------------- E2M1 ----

def test_e2m1_decode_is_the_grid():
    vals = [oracle.e2m1_decode(c) for c in range(16)]
    assert vals[:8] == E2M1_GRID
    assert vals[8:] == [-v for v in E2M1_GRID]
    assert np.signbit(vals[8])  # code 0x8 is -0


def test_e2m1_step_sizes_from_the_page():
    # Step 0.5 between 0 and 2, 1 between 2 and 4, 2 between 4 and 6.
    g = [oracle.e2m1_decode(c) for c in range(8)]
    steps = np.diff(g)
    assert list(steps[:4]) == [0.5] * 4
    assert list(steps[4:6]) == [1.0, 1.0]
    assert list(steps[6:]) == [2.0]


def _threshold_count(a):
    """E2M1 magnitude index by counting round-to-nearest-even decision points.

    Midpoints between neighbours are 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5; at a
    midpoint the even index wins, so the comparison is strict when the upper
    neighbour is odd and non-strict when it is even.
    """
    a = np.asarray(a, np.float32)
    m = ((a > 0.25).astype(np.uint8) + (a >= 0.75) + (a > 1.25) + (a >= 1.75)
         + (a > 2.5) + (a >= 3.5) + (a > 5.0))
    return m.astype(np.uint8)


def test_e2m1_encode_exhaustive_0_to_8():
    hi = int(f32_bits(8.0))
    step = 1 << 25
    for start in range(0, hi + 1, step):
        u = np.arange(start, min(start + step, hi + 1), dtype=np.uint32)
        a = from_bits(u)
        got = oracle.e2m1_index_array(a)
        want = _threshold_count(a)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (a[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_e2m1_encode_above_8_and_specials():
    rng = np.random.default_rng(3)
    u = rng.integers(int(f32_bits(8.0)), 0x7F800000, size=200000, dtype=np.uint64).astype(np.uint32)
    a = from_bits(u)
    assert (oracle.e2m1_index_array(a) == 7).all()
    assert oracle.e2m1_index(float("inf")) == 7
    assert oracle.e2m1_index(float("nan")) == 0
    assert oracle.e2m1_index(np.finfo(np.float32).max) == 7
    # the pages' worst case: scaled value 5 is the widest gap (between 4 and 6)
    assert oracle.e2m1_index(5.0) == 6 and oracle.e2m1_index(np.nextafter(np.float32(5), 6)) == 7


# ---------------------------------------------------------------- E4M3 ----

def _torch_e4m3(s):
    return torch.from_numpy(np.asarray(s, np.float32).copy()).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_e4m3_decode_matches_torch_all_bytes():
    b = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(b.copy()).view(torch.float8_e4m3fn).float().numpy()
    got = np.array([oracle.e4m3_decode(int(v)) for v in b], np.float32)
    same = (got.view(np.uint32) == want.view(np.uint32)) | (np.isnan(got) & np.isnan(want))
    assert same.all()
    assert oracle.e4m3_decode(0x7E) == 448.0
    assert oracle.e4m3_decode(0x01) == 2.0 ** -9


def test_e4m3_encode_matches_torch_near_every_decision_point():
    vals = np.array([oracle.e4m3_decode(S) for S in range(0x7F)], np.float64)
    mids = (vals[:-1] + vals[1:]) / 2  # exact in binary64, and in binary32
    pts = np.concatenate([vals, mids]).astype(np.float32)
    win = np.arange(-2048, 2049, dtype=np.int64)
    u = (f32_bits(pts).astype(np.int64)[:, None] + win[None, :]).reshape(-1)
    u = u[(u >= 0) & (u <= int(f32_bits(464.0)))].astype(np.uint32)
    s = from_bits(u)
    got = oracle.e4m3_encode_array(s)
    want = _torch_e4m3(s)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (s[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_e4m3_encode_matches_torch_random_patterns():
    rng = np.random.default_rng(11)
    u = rng.integers(0, int(f32_bits(464.0)) + 1, size=3_000_000, dtype=np.uint64).astype(np.uint32)
    s = from_bits(u)
    got = oracle.e4m3_encode_array(s)
    want = _torch_e4m3(s)
    assert (got == want).all()


def test_e4m3_encode_saturates_and_specials():
    rng = np.random.default_rng(5)
    u = rng.integers(int(f32_bits(464.0)) + 1, 0x7F800001, size=100000, dtype=np.uint64)
    s = from_bits(u.astype(np.uint32))
    assert (oracle.e4m3_encode_array(s) == 0x7E).all()  # saturating, never NaN
    assert oracle.e4m3_encode(0.0) == 0
    assert oracle.e4m3_encode(float("nan")) == 0
    assert oracle.e4m3_encode(2.0 ** -10) == 0  # tie between 0 and 2^-9 -> even
    assert oracle.e4m3_encode(float(np.nextafter(np.float32(2.0 ** -10), 1))) == 1
    assert oracle.e4m3_encode(448.0) == 0x7E


def _rn32(q: Fraction) -> np.float32:
    """Nearest binary32 to an exact rational, ties to even."""
    c = np.float32(float(q))
    best = None
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        dist = abs(Fraction(float(cand)) - q)
        key = (dist, int(np.float32(cand).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return np.float32(best[1])


def test_e4m3_reciprocal_table_is_correctly_rounded():
    assert oracle.e4m3_recip(0) == 0.0
    for S in range(1, 0x7F):
        want = _rn32(1 / Fraction(oracle.e4m3_decode(S)))
        got = np.float32(oracle.e4m3_recip(S))
        assert got.view(np.uint32) == want.view(np.uint32), S
