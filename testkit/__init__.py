"""Seeded synthetic inputs shared by the tests and the benchmark.

Holds no NVFP4 arithmetic: it draws random numbers (C, counter-based
SplitMix64) and rounds them to bf16.  The same host buffer feeds the oracle
and the GPU, so parity never depends on the host's libm.

The five workloads follow the statement of the benchmark configurations;
values are synthetic stand-ins for LLM activations, weights and gradients
with the outlier structure NVFP4 block scaling is meant to localise
("Why Gated DeltaNet in hybrid 27B LLMs withstands 4-bit quantization",
"Deep analysis").
"""
import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "synth.c")
LIB = os.path.join(HERE, "libsynth.so")

NORMAL, STUDENT_T3, LAPLACE, UNIFORM = 0, 1, 2, 3
MODE_STD, MODE_4OVER6 = 0, 1
RULE_MSE, RULE_MAE, RULE_MAX = 0, 1, 2
AXIS_ROWS, AXIS_COLS = 0, 1

GAMMA = 0x9E3779B97F4A7C15
_lib = None


def build():
    cmd = ["gcc", "-std=gnu99", "-O2", "-fPIC", "-Wall", "-shared", "-pthread", "-o", LIB, SRC, "-lm"]
    subprocess.run(cmd, check=True, cwd=HERE)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        P, i64, u64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64
        L.synth_fill.argtypes = [ctypes.c_int, ctypes.c_double, u64, i64, P, ctypes.c_int]
        L.synth_fill.restype = None
        L.synth_sample.argtypes = [u64, i64, i64, P]
        L.synth_sample.restype = i64
        L.synth_scale_at.argtypes = [P, P, i64, ctypes.c_double]
        L.synth_scale_at.restype = None
        L.synth_replace_laplace.argtypes = [P, P, i64, u64, ctypes.c_double]
        L.synth_replace_laplace.restype = None
        L.synth_scale_columns.argtypes = [P, i64, i64, P, i64, ctypes.c_double]
        L.synth_scale_columns.restype = None
        L.synth_fnv1a64.argtypes = [P, i64]
        L.synth_fnv1a64.restype = u64
        L.synth_draw.argtypes = [u64, u64]
        L.synth_draw.restype = u64
        _lib = L
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def default_threads():
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return max(1, min(16, os.cpu_count() or 1))


def fill(shape, dist=NORMAL, scale=1.0, seed=1, threads=None):
    """bf16 bit patterns (uint16) of scale * D for a seeded distribution D."""
    out = np.empty(shape, np.uint16)
    lib().synth_fill(int(dist), float(scale), seed & (2**64 - 1), out.size, _p(out),
                     threads or default_threads())
    return out


def sample(seed, n, k):
    """k distinct indices of range(n) (Floyd's algorithm), in draw order."""
    idx = np.empty(max(k, 1), np.int64)
    got = lib().synth_sample(seed & (2**64 - 1), int(n), int(k), _p(idx))
    if got != k:
        raise ValueError("bad sample arguments")
    return idx[:k]


def scale_at(x, idx, factor):
    idx = np.ascontiguousarray(idx, np.int64)
    lib().synth_scale_at(_p(x), _p(idx), idx.size, float(factor))


def replace_laplace(x, idx, seed, beta):
    idx = np.ascontiguousarray(idx, np.int64)
    lib().synth_replace_laplace(_p(x), _p(idx), idx.size, seed & (2**64 - 1), float(beta))


def scale_columns(x, cols_idx, factor):
    idx = np.ascontiguousarray(cols_idx, np.int64)
    rows, cols = x.shape
    lib().synth_scale_columns(_p(x), rows, cols, _p(idx), idx.size, float(factor))


def fnv1a64(a):
    a = np.ascontiguousarray(a)
    return int(lib().synth_fnv1a64(_p(a), a.nbytes))


@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    rows: int
    cols: int
    mode: int
    rule: int
    block_axis: int
    recipe: str

    @property
    def numel(self):
        return self.rows * self.cols


WORKLOADS = {
    1: Config(1, "std_256x1024_roundtrip", 256, 1024, MODE_STD, RULE_MSE, AXIS_COLS,
              "N(0,1); round(0.5% of N) = 1311 distinct seeded positions x50"),
    2: Config(2, "4over6_mse_4096x5120_act", 4096, 5120, MODE_4OVER6, RULE_MSE, AXIS_COLS,
              "N(0,1); 4 distinct seeded columns x60"),
    3: Config(3, "4over6_mae_17408x5120_weight", 17408, 5120, MODE_4OVER6, RULE_MAE, AXIS_COLS,
              "0.02*N(0,1); round(0.1% of N) = 89129 distinct positions replaced by Laplace(0,0.2)"),
    4: Config(4, "4over6_mse_32768x5120_prefill", 32768, 5120, MODE_4OVER6, RULE_MSE, AXIS_COLS,
              "0.5*Student-t(3); 8 distinct seeded columns x100; bitmap + per-tensor MSE"),
    5: Config(5, "4over6_mae_8192x5120_grad_colblocked", 8192, 5120, MODE_4OVER6, RULE_MAE,
              AXIS_ROWS, "1e-4*N(0,1); round(1% of N) = 419430 distinct positions x30"),
}


def seeds(cid):
    values = 0x4F36000000000000 + cid
    return values, values ^ GAMMA, values ^ 0xD1B54A32D192ED03


def make(cid, rows=None, cols=None, threads=None):
    """The bf16 tensor of workload `cid` (optionally at another shape with the
    same recipe: outlier counts scale with the element count)."""
    cfg = WORKLOADS[cid]
    rows = rows or cfg.rows
    cols = cols or cfg.cols
    n = rows * cols
    s_val, s_pos, s_lap = seeds(cid)
    if cid == 1:
        x = fill((rows, cols), NORMAL, 1.0, s_val, threads)
        scale_at(x.reshape(-1), sample(s_pos, n, int(round(0.005 * n))), 50.0)
    elif cid == 2:
        x = fill((rows, cols), NORMAL, 1.0, s_val, threads)
        scale_columns(x, sample(s_pos, cols, 4), 60.0)
    elif cid == 3:
        x = fill((rows, cols), NORMAL, 0.02, s_val, threads)
        replace_laplace(x.reshape(-1), sample(s_pos, n, int(round(0.001 * n))), s_lap, 0.2)
    elif cid == 4:
        x = fill((rows, cols), STUDENT_T3, 0.5, s_val, threads)
        scale_columns(x, sample(s_pos, cols, 8), 100.0)
    elif cid == 5:
        x = fill((rows, cols), NORMAL, 1e-4, s_val, threads)
        scale_at(x.reshape(-1), sample(s_pos, n, int(round(0.01 * n))), 30.0)
    else:
        raise KeyError(cid)
    return x


def bf16_to_f32(x_bf16):
    """Exact widening of bf16 bit patterns to float32 values."""
    return (np.asarray(x_bf16, np.uint16).astype(np.uint32) << 16).view(np.float32)
