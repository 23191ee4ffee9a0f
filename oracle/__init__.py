"""ctypes binding of the CPU oracle.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
CPU-baseline leg of the benchmark, never by the product library.  The oracle
shares no code with the HIP path.
"""
import ctypes
import os

import numpy as np

from . import build as _build

MODE_STD, MODE_4OVER6 = 0, 1
RULE_MSE, RULE_MAE, RULE_MAX = 0, 1, 2
AXIS_ROWS, AXIS_COLS = 0, 1

_lib = None


class BlockDetail(ctypes.Structure):
    _fields_ = [
        ("b", ctypes.c_float),
        ("ncand", ctypes.c_int),
        ("k", ctypes.c_float * 2),
        ("s", ctypes.c_float * 2),
        ("S", ctypes.c_uint8 * 2),
        ("d", ctypes.c_float * 2),
        ("r", ctypes.c_float * 2),
        ("y", (ctypes.c_float * 16) * 2),
        ("code", (ctypes.c_uint8 * 16) * 2),
        ("xhat", (ctypes.c_float * 16) * 2),
        ("delta", (ctypes.c_float * 16) * 2),
        ("err", ctypes.c_float * 2),
        ("chosen", ctypes.c_int),
    ]


def lib():
    """Load the oracle library, compiling it first only if it is not built."""
    global _lib
    if _lib is None:
        path = os.environ.get("NVFP4_ORACLE_LIB")  # e.g. the sanitizer build
        if not path:
            path = _build.LIB
            if not os.path.exists(path):
                _build.build()
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        L.nvfp4o_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.nvfp4o_bf16_to_f32.restype = ctypes.c_float
        L.nvfp4o_f32_to_bf16.argtypes = [ctypes.c_float]
        L.nvfp4o_f32_to_bf16.restype = ctypes.c_uint16
        L.nvfp4o_e2m1_index.argtypes = [ctypes.c_float]
        L.nvfp4o_e2m1_index.restype = ctypes.c_int
        L.nvfp4o_e2m1_decode.argtypes = [ctypes.c_uint8]
        L.nvfp4o_e2m1_decode.restype = ctypes.c_float
        L.nvfp4o_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.nvfp4o_e4m3_decode.restype = ctypes.c_float
        L.nvfp4o_e4m3_encode.argtypes = [ctypes.c_float]
        L.nvfp4o_e4m3_encode.restype = ctypes.c_uint8
        L.nvfp4o_e4m3_recip.argtypes = [ctypes.c_uint8]
        L.nvfp4o_e4m3_recip.restype = ctypes.c_float
        L.nvfp4o_e2m1_index_array.argtypes = [P, i64, P]
        L.nvfp4o_e2m1_index_array.restype = None
        L.nvfp4o_e4m3_encode_array.argtypes = [P, i64, P]
        L.nvfp4o_e4m3_encode_array.restype = None
        L.nvfp4o_amax.argtypes = [P, i64]
        L.nvfp4o_amax.restype = ctypes.c_float
        L.nvfp4o_global_scale.argtypes = [ctypes.c_float, ctypes.c_int]
        L.nvfp4o_global_scale.restype = ctypes.c_float
        L.nvfp4o_quantize_block.argtypes = [P, ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                            ctypes.POINTER(BlockDetail)]
        L.nvfp4o_quantize_block.restype = None
        L.nvfp4o_quantize.argtypes = [P, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, P, P, P, P, P]
        L.nvfp4o_quantize.restype = ctypes.c_int
        L.nvfp4o_quantize_mt.argtypes = [P, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, P, P, P, P, P]
        L.nvfp4o_quantize_mt.restype = ctypes.c_int
        L.nvfp4o_dequantize.argtypes = [P, P, ctypes.c_float, i64, i64, ctypes.c_int,
                                        ctypes.c_int, P]
        L.nvfp4o_dequantize.restype = ctypes.c_int
        L.nvfp4o_channel_absmax.argtypes = [P, i64, i64, P]
        L.nvfp4o_channel_absmax.restype = None
        L.nvfp4o_channel_order.argtypes = [P, i64, P]
        L.nvfp4o_channel_order.restype = None
        L.nvfp4o_quantize_residual.argtypes = [P, i64, i64, P, i64, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int, P, P, P]
        L.nvfp4o_quantize_residual.restype = ctypes.c_int
        L.nvfp4o_quantize_augmented.argtypes = [P, i64, i64, P, i64, ctypes.c_int, ctypes.c_int,
                                                ctypes.c_int, P, P, P, ctypes.c_int]
        L.nvfp4o_quantize_augmented.restype = ctypes.c_int
        L.nvfp4o_gemm.argtypes = [P, P, ctypes.c_float, P, P, ctypes.c_float, i64, i64, i64, P, P]
        L.nvfp4o_gemm.restype = ctypes.c_int
        L.nvfp4o_rms_rstd.argtypes = [P, i64, ctypes.c_float]
        L.nvfp4o_rms_rstd.restype = ctypes.c_float
        L.nvfp4o_rmsnorm.argtypes = [P, i64, i64, P, ctypes.c_float, P]
        L.nvfp4o_rmsnorm.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


# --- scalar codecs --------------------------------------------------------

def e2m1_index(a):
    return lib().nvfp4o_e2m1_index(float(a))


def e2m1_decode(code):
    return lib().nvfp4o_e2m1_decode(int(code))


def e4m3_decode(S):
    return lib().nvfp4o_e4m3_decode(int(S))


def e4m3_encode(s):
    return lib().nvfp4o_e4m3_encode(float(s))


def e4m3_recip(S):
    return lib().nvfp4o_e4m3_recip(int(S))


def e2m1_index_array(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, np.uint8)
    lib().nvfp4o_e2m1_index_array(_ptr(a), a.size, _ptr(out))
    return out


def e4m3_encode_array(s):
    s = np.ascontiguousarray(s, dtype=np.float32)
    out = np.empty(s.shape, np.uint8)
    lib().nvfp4o_e4m3_encode_array(_ptr(s), s.size, _ptr(out))
    return out


def bf16_to_f32(h):
    return lib().nvfp4o_bf16_to_f32(int(h))


def f32_to_bf16(f):
    return lib().nvfp4o_f32_to_bf16(float(f))


# --- tensors ----------------------------------------------------------------

def amax(x_bf16):
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    return np.float32(lib().nvfp4o_amax(_ptr(x), x.size))


def global_scale(a, mode):
    return np.float32(lib().nvfp4o_global_scale(float(a), int(mode)))


def quantize_block(x16, g, mode, rule):
    """Quantize one block of 16 fp32 values; returns the full BlockDetail."""
    x = np.ascontiguousarray(x16, dtype=np.float32)
    assert x.size == 16
    out = BlockDetail()
    lib().nvfp4o_quantize_block(_ptr(x), float(np.float32(g)), int(mode), int(rule),
                                ctypes.byref(out))
    return out


def output_shapes(rows, cols, block_axis):
    """Byte sizes of (packed, scales, selmap) for a [rows][cols] tensor."""
    n = rows * cols
    nblocks = n // 16
    return n // 2, nblocks, (nblocks + 7) // 8


def quantize(x_bf16, block_axis, mode, rule, gscale=None, want_selmap=True, want_err=True):
    """Quantize a [rows][cols] bf16 tensor (uint16 bit patterns).

    Returns dict(packed, scales, gscale, selmap, err_sum).  For block_axis
    AXIS_ROWS the packed/scales/selmap arrays are in the layout of the
    transposed tensor.
    """
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, cols = x.shape
    n_packed, n_scales, n_sel = output_shapes(rows, cols, block_axis)
    packed = np.zeros(n_packed, np.uint8)
    scales = np.zeros(n_scales, np.uint8)
    selmap = np.zeros(n_sel, np.uint8) if want_selmap else None
    err = np.zeros(1, np.float64) if want_err else None
    g = np.zeros(1, np.float32)
    given = 0
    if gscale is not None:
        g[0] = np.float32(gscale)
        given = 1
    st = lib().nvfp4o_quantize(_ptr(x), rows, cols, int(block_axis), int(mode), int(rule), given,
                               _ptr(g), _ptr(packed), _ptr(scales), _ptr(selmap), _ptr(err))
    if st != 0:
        raise ValueError(f"oracle quantize failed with status {st}")
    return {
        "packed": packed,
        "scales": scales,
        "gscale": np.float32(g[0]),
        "selmap": selmap,
        "err_sum": float(err[0]) if want_err else None,
    }


def quantize_mt(x_bf16, mode, rule, threads, gscale=None):
    """quantize(x, AXIS_COLS, ...) run on `threads` host threads (the CPU
    baseline's driver); bit-identical outputs."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, cols = x.shape
    n_packed, n_scales, n_sel = output_shapes(rows, cols, AXIS_COLS)
    packed = np.zeros(n_packed, np.uint8)
    scales = np.zeros(n_scales, np.uint8)
    selmap = np.zeros(n_sel, np.uint8)
    err = np.zeros(1, np.float64)
    g = np.zeros(1, np.float32)
    given = 0
    if gscale is not None:
        g[0] = np.float32(gscale)
        given = 1
    st = lib().nvfp4o_quantize_mt(_ptr(x), rows, cols, int(mode), int(rule), int(threads),
                                  given, _ptr(g), _ptr(packed), _ptr(scales), _ptr(selmap),
                                  _ptr(err))
    if st != 0:
        raise ValueError(f"oracle quantize_mt failed with status {st}")
    return {"packed": packed, "scales": scales, "gscale": np.float32(g[0]), "selmap": selmap,
            "err_sum": float(err[0])}


def dequantize(packed, scales, gscale, rows, cols, block_axis, out_bf16=False):
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    s = np.ascontiguousarray(scales, dtype=np.uint8)
    out = np.zeros((rows, cols), np.uint16 if out_bf16 else np.float32)
    st = lib().nvfp4o_dequantize(_ptr(p), _ptr(s), float(np.float32(gscale)), rows, cols,
                                 int(block_axis), int(bool(out_bf16)), _ptr(out))
    if st != 0:
        raise ValueError(f"oracle dequantize failed with status {st}")
    return out


# --- residual channels --------------------------------------------------------

def channel_absmax(x_bf16):
    """absmax[c] = max over rows of |x[r][c]| for a [rows][cols] bf16 tensor."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, cols = x.shape
    out = np.zeros(cols, np.float32)
    lib().nvfp4o_channel_absmax(_ptr(x), rows, cols, _ptr(out))
    return out


def channel_order(absmax):
    """Channel order by absolute maximum, largest first, ties by lower index."""
    a = np.ascontiguousarray(absmax, dtype=np.float32)
    perm = np.zeros(a.size, np.int32)
    lib().nvfp4o_channel_order(_ptr(a), a.size, _ptr(perm))
    return perm


def quantize_residual(x_bf16, perm, nres, mode, rule, gscale=None, duplicate=False):
    """Two-stage quantization with reordered channels and nres residual channels.

    duplicate=True gives the weight side of the augmented product instead: the
    appended blocks repeat the primary blocks of the first nres positions.
    Returns dict(packed [rows][(cols+nres)/2], scales [rows][(cols+nres)/16],
    gscale).
    """
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, cols = x.shape
    pm = np.ascontiguousarray(perm, dtype=np.int32)
    width = cols + int(nres)
    packed = np.zeros((rows, max(width, 0) // 2), np.uint8)
    scales = np.zeros((rows, max(width, 0) // 16), np.uint8)
    g = np.zeros(1, np.float32)
    given = 0
    if gscale is not None:
        g[0] = np.float32(gscale)
        given = 1
    st = lib().nvfp4o_quantize_augmented(_ptr(x), rows, cols, _ptr(pm), int(nres), int(mode),
                                         int(rule), given, _ptr(g), _ptr(packed), _ptr(scales),
                                         int(bool(duplicate)))
    if st != 0:
        raise ValueError(f"oracle quantize_residual failed with status {st}")
    return {"packed": packed, "scales": scales, "gscale": np.float32(g[0])}


def rms_rstd(xrow_bf16, eps):
    x = np.ascontiguousarray(xrow_bf16, dtype=np.uint16)
    return np.float32(lib().nvfp4o_rms_rstd(_ptr(x), x.size, float(np.float32(eps))))


def rmsnorm(x_bf16, weight_bf16, eps):
    """RMSNorm of a [rows][cols] bf16 tensor as the fused path defines it;
    returns bf16 bit patterns (uint16)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, cols = x.shape
    w = None if weight_bf16 is None else np.ascontiguousarray(weight_bf16, dtype=np.uint16)
    y = np.zeros((rows, cols), np.uint16)
    st = lib().nvfp4o_rmsnorm(_ptr(x), rows, cols, _ptr(w), float(np.float32(eps)), _ptr(y))
    if st != 0:
        raise ValueError(f"oracle rmsnorm failed with status {st}")
    return y


def gemm(a_packed, a_scales, ga, b_packed, b_scales, gb, M, N, K, want_abs=False):
    """W4A4 product of two NVFP4 tensors blocked along K (AXIS_COLS layout):
    out [M][N] = ga * gb * sum_k a(m,k) b(n,k) in binary64, and with want_abs
    also ga * gb * sum_k |a(m,k) b(n,k)|.  Returns out or (out, abs)."""
    pa = np.ascontiguousarray(a_packed, dtype=np.uint8)
    sa = np.ascontiguousarray(a_scales, dtype=np.uint8)
    pb = np.ascontiguousarray(b_packed, dtype=np.uint8)
    sb = np.ascontiguousarray(b_scales, dtype=np.uint8)
    M, N, K = int(M), int(N), int(K)
    if K % 16 or pa.size != M * K // 2 or sa.size != M * K // 16 or \
            pb.size != N * K // 2 or sb.size != N * K // 16:
        raise ValueError("gemm: operand sizes do not match M, N, K")
    out = np.zeros((M, N), np.float64)
    aout = np.zeros((M, N), np.float64) if want_abs else None
    st = lib().nvfp4o_gemm(_ptr(pa), _ptr(sa), float(np.float32(ga)), _ptr(pb), _ptr(sb),
                           float(np.float32(gb)), M, N, K, _ptr(out),
                           _ptr(aout) if want_abs else None)
    if st != 0:
        raise ValueError(f"oracle gemm failed with status {st}")
    return (out, aout) if want_abs else out
