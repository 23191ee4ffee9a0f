"""Python binding of the NVFP4 / Four-Over-Six C ABI (include/nvfp4.h).

Argument marshalling only: every step of quantization runs in the HIP
library built from csrc/ for gfx950.  There is no fallback; if the library
is missing or was not built, every call raises.  PyTorch supplies device
memory and streams.

Format and method: 16-element blocks with FP8 E4M3 scales, E2M1 codes and an
fp32 tensor scale; under 4/6 each block is quantized with its max mapped to 6
and to 4 and the one with lower MSE/MAE is kept ("Technical summary: Four
Over Six (4/6)", gist.science 2512.02010, "Adaptive block scaling
algorithm" and "Implementation details").
"""
import ctypes
import math
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnvfp4.so")

AXIS_ROWS, AXIS_COLS = 0, 1
MODE_STD, MODE_4OVER6 = 0, 1
RULE_MSE, RULE_MAE, RULE_MAX = 0, 1, 2
OUT_F32, OUT_BF16 = 0, 1
FLAG_GSCALE_GIVEN = 1
FLAG_ERR_ACCUMULATE = 2
FLAG_STATS_ACCUMULATE = 4
FLAG_RESIDUAL_DUPLICATE = 8

STATUS = {0: "NVFP4_OK", 1: "NVFP4_ERR_NULL", 2: "NVFP4_ERR_ENUM", 3: "NVFP4_ERR_SHAPE",
          4: "NVFP4_ERR_ALIGN", 5: "NVFP4_ERR_HIP", 6: "NVFP4_ERR_ALIAS", 7: "NVFP4_ERR_SCRATCH"}
# Largest splits * M * N of nvfp4_gemm_splitk_noalloc (its fixed scratch).
NOALLOC_SCRATCH_FLOATS = 1 << 23

# Every symbol the public headers declare, with its ctypes signature.
_P, _I64, _I, _U32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint32
SIGNATURES = {
    "nvfp4_amax": ([_P, _I64, _P, _P], _I),
    "nvfp4_global_scale": ([_P, _I, _P, _P], _I),
    "nvfp4_quantize": ([_P, _I64, _I64, _I, _I, _I, _P, _P, _P, _P], _I),
    "nvfp4_quantize_ex": ([_P, _I64, _I64, _I, _I, _I, _U32, _P, _P, _P, _P, _P, _P], _I),
    "nvfp4_quantize_ex_timed": ([_P, _I64, _I64, _I, _I, _I, _U32, _P, _P, _P, _P, _P, _P, _P,
                                 _P], _I),
    "nvfp4_quantize_delayed": ([_P, _I64, _I64, _I, _I, _I, _U32, _P, _P, _P, _P, _P, _P, _P],
                               _I),
    "nvfp4_quantize_dual": ([_P, _I64, _I64, _I, _I, _U32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
                            _I),
    "nvfp4_dequantize": ([_P, _P, _P, _I64, _I64, _I, _I, _P, _P], _I),
    "nvfp4_channel_order": ([_P, _I64, _I64, _U32, _P, _P, _P], _I),
    "nvfp4_check_order": ([_P, _I64, _P, _P], _I),
    "nvfp4_quantize_residual": ([_P, _I64, _I64, _P, _I64, _I, _I, _U32, _P, _P, _P, _P], _I),
    "nvfp4_rmsnorm_quantize_residual": ([_P, _I64, _I64, _P, ctypes.c_float, _P, _I64, _I, _I,
                                         _U32, _P, _P, _P, _P, _P], _I),
    "nvfp4_gemm": ([_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _P, _P], _I),
    "nvfp4_gemm_splitk": ([_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _I, _P, _P, _I64, _P],
                          _I),
    "nvfp4_gemm_splitk_noalloc": ([_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _I, _P, _P],
                                  _I),
    "nvfp4_gemm_splits_hint": ([_I64, _I64, _I64], _I),
    "nvfp4_status_string": ([_I], ctypes.c_char_p),
    "nvfp4v_e2m1_encode_sweep": ([_U32, _I64, _P, _P], _I),
    "nvfp4v_e4m3_encode_sweep": ([_U32, _I64, _P, _P], _I),
    "nvfp4v_decode_tables": ([ctypes.c_float, _P, _P, _P, _P, _P], _I),
    "nvfp4v_stream_pattern": ([_P, _I64, _P, _P, _P], _I),
}


class NVFP4Error(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({_status_text(status)})")


_lib = None


def lib():
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run nvfp4_block_scaled_wave64_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _status_text(status):
    try:
        return lib().nvfp4_status_string(int(status)).decode()
    except Exception:  # pragma: no cover
        return "?"


def _check(status, what):
    if status != 0:
        raise NVFP4Error(status, what)


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _bf16_input(x):
    if x.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError("input must hold bf16 bit patterns (bfloat16, int16 or uint16)")
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError("input must be a contiguous device tensor")
    return x


def _need(t, numel, dtype, dev, name):
    """t, checked to be a contiguous `dtype` tensor on `dev` holding at least
    `numel` elements (what the library reads or writes there)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype or t.device != dev or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous {dtype} tensor on {dev}")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements; {numel} are needed")
    return t


def _out(out, key, shape, dtype, dev):
    """out[key] checked against `shape`, or a new tensor of that shape."""
    t = out.get(key)
    if t is None:
        return torch.empty(shape, dtype=dtype, device=dev)
    return _need(t, math.prod(shape), dtype, dev, f"out[{key!r}]")


def output_shapes(rows, cols, block_axis):
    """Shapes of (packed, scales) and the bitmap length for a [rows][cols] tensor."""
    n_rows, n_cols = (rows, cols) if block_axis == AXIS_COLS else (cols, rows)
    nblocks = rows * cols // 16
    return (n_rows, n_cols // 2), (n_rows, n_cols // 16), (nblocks + 7) // 8


def amax(x, out=None, stream=None):
    """A = max |x| of a bf16 tensor, as a 1-element float32 device tensor."""
    x = _bf16_input(x)
    out = _out({"amax": out}, "amax", (1,), torch.float32, x.device)
    _check(lib().nvfp4_amax(_ptr(x), x.numel(), _ptr(out), _stream(stream)), "nvfp4_amax")
    return out


def global_scale(amax_t, mode, out=None, stream=None):
    """g = A / (6*M) (M = 448 standard, 256 under 4/6) from a device amax."""
    dev = amax_t.device
    amax_t = _need(amax_t, 1, torch.float32, dev, "amax")
    out = _out({"gscale": out}, "gscale", (1,), torch.float32, dev)
    _check(lib().nvfp4_global_scale(_ptr(amax_t), int(mode), _ptr(out), _stream(stream)),
           "nvfp4_global_scale")
    return out


def _event_handle(ev, stream):
    """Raw hipEvent_t of a timing torch.cuda.Event (created on first use by
    recording it once on `stream`), or an integer handle as given."""
    if isinstance(ev, torch.cuda.Event):
        if not ev.cuda_event:
            ev.record(stream)
        return ctypes.c_void_p(ev.cuda_event)
    return ctypes.c_void_p(int(ev)) if ev else None


def quantize(x, block_axis=AXIS_COLS, mode=MODE_4OVER6, rule=RULE_MSE, gscale=None,
             selmap=False, err_sum=False, err_accumulate=False, out=None, stream=None,
             events=None):
    """Quantize a [rows][cols] bf16 device tensor.

    gscale: optional 1-element float32 device tensor holding a given g (the
    amax pass is skipped).  Returns a dict with packed, scales, gscale and,
    when asked for, selmap (uint8 bitmap) and err_sum (float64, 1 element).
    err_accumulate adds the error sum to out["err_sum"] instead of zeroing it
    first.  `out` may supply preallocated tensors under the same keys.
    events: optional (start, stop) pair of timing torch.cuda.Event objects
    (or raw hipEvent_t handles) bound to the quantization kernels themselves
    (nvfp4_quantize_ex_timed): start.elapsed_time(stop) is their execution
    time without the amax pass or dispatch gaps.
    """
    x = _bf16_input(x)
    if x.dim() != 2:
        raise ValueError("input must be 2-D [rows][cols]")
    rows, cols = x.shape
    pshape, sshape, nsel = output_shapes(rows, cols, block_axis)
    dev = x.device
    out = dict(out or {})
    packed = _out(out, "packed", pshape, torch.uint8, dev)
    scales = _out(out, "scales", sshape, torch.uint8, dev)
    flags = 0
    if gscale is not None:
        g = _need(gscale, 1, torch.float32, dev, "gscale")
        flags |= FLAG_GSCALE_GIVEN
    else:
        g = _out(out, "gscale", (1,), torch.float32, dev)
    sel = _out(out, "selmap", (max(nsel, 1),), torch.uint8, dev) if selmap else None
    if err_sum and err_accumulate and out.get("err_sum") is None:
        raise ValueError("err_accumulate needs out['err_sum']")
    err = _out(out, "err_sum", (1,), torch.float64, dev) if err_sum else None
    if err_sum and err_accumulate:
        flags |= FLAG_ERR_ACCUMULATE
    args = (_ptr(x), rows, cols, int(block_axis), int(mode), int(rule), flags, _ptr(packed),
            _ptr(scales), _ptr(g), _ptr(sel), _ptr(err))
    if events is None:
        _check(lib().nvfp4_quantize_ex(*args, _stream(stream)), "nvfp4_quantize_ex")
    else:
        st = stream if stream is not None else torch.cuda.current_stream()
        ev0, ev1 = (_event_handle(e, st) for e in events)
        _check(lib().nvfp4_quantize_ex_timed(*args, ev0, ev1, _stream(stream)),
               "nvfp4_quantize_ex_timed")
    res = {"packed": packed, "scales": scales, "gscale": g}
    if selmap:
        res["selmap"] = sel
    if err_sum:
        res["err_sum"] = err
    return res


def quantize_dual(x, mode=MODE_4OVER6, rule=RULE_MSE, gscale=None, selmap=False, err_sum=False,
                  err_accumulate=False, out=None, stream=None):
    """Both block layouts of a [rows][cols] bf16 tensor from one read
    (nvfp4_quantize_dual).  Returns {"gscale": g, "rows": {...}, "cols": {...}}
    where "rows" holds the row-blocked outputs (those of quantize with
    AXIS_COLS) and "cols" the column-blocked ones (AXIS_ROWS): packed,
    scales and, when asked for, selmap and err_sum.  `out` may supply
    {"gscale": ..., "rows": {...}, "cols": {...}} tensors."""
    x = _bf16_input(x)
    if x.dim() != 2:
        raise ValueError("input must be 2-D [rows][cols]")
    rows, cols = x.shape
    dev = x.device
    out = dict(out or {})
    sides = {}
    for key, axis in (("rows", AXIS_COLS), ("cols", AXIS_ROWS)):
        pshape, sshape, nsel = output_shapes(rows, cols, axis)
        o = dict(out.get(key) or {})
        d = {"packed": _out(o, "packed", pshape, torch.uint8, dev),
             "scales": _out(o, "scales", sshape, torch.uint8, dev)}
        if selmap:
            d["selmap"] = _out(o, "selmap", (max(nsel, 1),), torch.uint8, dev)
        if err_sum:
            if err_accumulate and o.get("err_sum") is None:
                raise ValueError("err_accumulate needs out[side]['err_sum']")
            d["err_sum"] = _out(o, "err_sum", (1,), torch.float64, dev)
        sides[key] = d
    flags = 0
    if gscale is not None:
        g = _need(gscale, 1, torch.float32, dev, "gscale")
        flags |= FLAG_GSCALE_GIVEN
    else:
        g = _out(out, "gscale", (1,), torch.float32, dev)
    if err_sum and err_accumulate:
        flags |= FLAG_ERR_ACCUMULATE
    r, c = sides["rows"], sides["cols"]
    st = lib().nvfp4_quantize_dual(_ptr(x), rows, cols, int(mode), int(rule), flags,
                                   _ptr(r["packed"]), _ptr(r["scales"]), _ptr(c["packed"]),
                                   _ptr(c["scales"]), _ptr(g), _ptr(r.get("selmap")),
                                   _ptr(c.get("selmap")), _ptr(r.get("err_sum")),
                                   _ptr(c.get("err_sum")), _stream(stream))
    _check(st, "nvfp4_quantize_dual")
    return {"gscale": g, "rows": r, "cols": c}


def quantize_delayed(x, gscale, block_axis=AXIS_COLS, mode=MODE_4OVER6, rule=RULE_MSE,
                     selmap=False, err_sum=False, err_accumulate=False, out=None, stream=None):
    """Quantize with a given tensor scale g (1-element float32 device tensor,
    e.g. global_scale(previous amax)) and record this tensor's amax in the
    same pass (nvfp4_quantize_delayed).  Returns the dict of quantize() with
    "amax" (1-element float32) in place of "gscale"."""
    x = _bf16_input(x)
    if x.dim() != 2:
        raise ValueError("input must be 2-D [rows][cols]")
    rows, cols = x.shape
    pshape, sshape, nsel = output_shapes(rows, cols, block_axis)
    dev = x.device
    out = dict(out or {})
    packed = _out(out, "packed", pshape, torch.uint8, dev)
    scales = _out(out, "scales", sshape, torch.uint8, dev)
    amax_t = _out(out, "amax", (1,), torch.float32, dev)
    sel = _out(out, "selmap", (max(nsel, 1),), torch.uint8, dev) if selmap else None
    if err_sum and err_accumulate and out.get("err_sum") is None:
        raise ValueError("err_accumulate needs out['err_sum']")
    err = _out(out, "err_sum", (1,), torch.float64, dev) if err_sum else None
    flags = FLAG_ERR_ACCUMULATE if (err_sum and err_accumulate) else 0
    st = lib().nvfp4_quantize_delayed(_ptr(x), rows, cols, int(block_axis), int(mode), int(rule),
                                      flags, _ptr(packed), _ptr(scales), _ptr(gscale),
                                      _ptr(amax_t), _ptr(sel), _ptr(err), _stream(stream))
    _check(st, "nvfp4_quantize_delayed")
    res = {"packed": packed, "scales": scales, "amax": amax_t}
    if selmap:
        res["selmap"] = sel
    if err_sum:
        res["err_sum"] = err
    return res


def channel_order(x, absmax=None, accumulate=False, perm=None, stream=None):
    """Channel statistic and order of a [rows][cols] bf16 activation tensor
    (nvfp4_channel_order): absmax[c] = max_r |x[r][c]| (float32, cols) and
    perm (int32, cols), the channels by decreasing absmax, ties by index.
    accumulate folds this tensor's maxima into the given `absmax` (a running
    maximum over calibration batches).  Returns (absmax, perm)."""
    x = _bf16_input(x)
    if x.dim() != 2:
        raise ValueError("input must be 2-D [rows][cols]")
    rows, cols = x.shape
    if absmax is None and accumulate:
        raise ValueError("accumulate needs absmax")
    absmax = _out({"absmax": absmax}, "absmax", (cols,), torch.float32, x.device)
    perm = _out({"perm": perm}, "perm", (cols,), torch.int32, x.device)
    flags = FLAG_STATS_ACCUMULATE if accumulate else 0
    _check(lib().nvfp4_channel_order(_ptr(x), rows, cols, flags, _ptr(absmax), _ptr(perm),
                                     _stream(stream)), "nvfp4_channel_order")
    return absmax, perm


def check_order(perm, stream=None):
    """nvfp4_check_order: the number of entries keeping the int32 device
    tensor `perm` from being a permutation of [0, len(perm)) (0: a valid
    channel order), as a 1-element int32 device tensor holding the call's
    uint32 count (read it after a synchronization)."""
    if not isinstance(perm, torch.Tensor) or perm.dim() != 1:
        raise ValueError("perm must be a 1-D int32 device tensor")
    perm = _need(perm, perm.numel(), torch.int32, perm.device, "perm")
    bad = torch.empty(1, dtype=torch.int32, device=perm.device)
    _check(lib().nvfp4_check_order(_ptr(perm), perm.numel(), _ptr(bad), _stream(stream)),
           "nvfp4_check_order")
    return bad


def quantize_residual(x, perm, nres, mode=MODE_4OVER6, rule=RULE_MSE, gscale=None, out=None,
                      stream=None, duplicate=False):
    """Two-stage quantization with reordered channels
    (nvfp4_quantize_residual).  perm: int32 device tensor of cols channel
    indices; nres: residual channels (multiple of 16, <= cols).  Returns a
    dict with packed [rows][(cols+nres)/2], scales [rows][(cols+nres)/16] and
    gscale; `gscale` given skips the amax pass.  duplicate=True quantizes the
    weight side of the augmented product (the appended blocks repeat the
    primary blocks of the first nres channels)."""
    x = _bf16_input(x)
    if x.dim() != 2:
        raise ValueError("input must be 2-D [rows][cols]")
    rows, cols = x.shape
    width = cols + int(nres)
    dev = x.device
    perm = _need(perm, cols, torch.int32, dev, "perm")
    out = dict(out or {})
    packed = _out(out, "packed", (rows, max(width, 0) // 2), torch.uint8, dev)
    scales = _out(out, "scales", (rows, max(width, 0) // 16), torch.uint8, dev)
    flags = FLAG_RESIDUAL_DUPLICATE if duplicate else 0
    if gscale is not None:
        g = _need(gscale, 1, torch.float32, dev, "gscale")
        flags |= FLAG_GSCALE_GIVEN
    else:
        g = _out(out, "gscale", (1,), torch.float32, dev)
    st = lib().nvfp4_quantize_residual(_ptr(x), rows, cols, _ptr(perm), int(nres), int(mode),
                                       int(rule), flags, _ptr(packed), _ptr(scales), _ptr(g),
                                       _stream(stream))
    _check(st, "nvfp4_quantize_residual")
    return {"packed": packed, "scales": scales, "gscale": g}


def rmsnorm_quantize_residual(x, perm, nres, weight=None, eps=1e-6, mode=MODE_4OVER6,
                              rule=RULE_MSE, gscale=None, amax=False, out=None, stream=None):
    """RMSNorm, channel reordering and the two quantization stages in one pass
    over x (nvfp4_rmsnorm_quantize_residual).  weight: bf16 device tensor of
    cols values, or None.  Returns the dict of quantize_residual, plus
    "amax" (max |y|, 1-element float32) when asked for."""
    x = _bf16_input(x)
    if x.dim() != 2:
        raise ValueError("input must be 2-D [rows][cols]")
    rows, cols = x.shape
    width = cols + int(nres)
    dev = x.device
    perm = _need(perm, cols, torch.int32, dev, "perm")
    if weight is not None:
        weight = _bf16_input(weight)
        if weight.numel() < cols or weight.device != dev:
            raise ValueError(f"weight must hold {cols} bf16 values on {dev}")
    out = dict(out or {})
    packed = _out(out, "packed", (rows, max(width, 0) // 2), torch.uint8, dev)
    scales = _out(out, "scales", (rows, max(width, 0) // 16), torch.uint8, dev)
    flags = 0
    if gscale is not None:
        g = _need(gscale, 1, torch.float32, dev, "gscale")
        flags |= FLAG_GSCALE_GIVEN
    else:
        g = _out(out, "gscale", (1,), torch.float32, dev)
    a = None
    if amax:
        a = _out(out, "amax", (1,), torch.float32, dev)
    st = lib().nvfp4_rmsnorm_quantize_residual(_ptr(x), rows, cols, _ptr(weight), float(eps),
                                               _ptr(perm), int(nres), int(mode), int(rule), flags,
                                               _ptr(packed), _ptr(scales), _ptr(g), _ptr(a),
                                               _stream(stream))
    _check(st, "nvfp4_rmsnorm_quantize_residual")
    res = {"packed": packed, "scales": scales, "gscale": g}
    if amax:
        res["amax"] = a
    return res


def dequantize(packed, scales, gscale, rows, cols, block_axis=AXIS_COLS, out_dtype=torch.float32,
               out=None, stream=None):
    """x_hat [rows][cols] (float32 or bfloat16) from packed codes and scales."""
    code = {torch.float32: OUT_F32, torch.bfloat16: OUT_BF16}[out_dtype]
    dev = packed.device
    packed = _need(packed, rows * cols // 2, torch.uint8, dev, "packed")
    scales = _need(scales, rows * cols // 16, torch.uint8, dev, "scales")
    gscale = _need(gscale, 1, torch.float32, dev, "gscale")
    out = _out({"out": out}, "out", (rows, cols), out_dtype, dev)
    st = lib().nvfp4_dequantize(_ptr(packed), _ptr(scales), _ptr(gscale), int(rows), int(cols),
                                int(block_axis), code, _ptr(out), _stream(stream))
    _check(st, "nvfp4_dequantize")
    return out


def gemm_splits_hint(M, N, K):
    """Split count nvfp4_gemm_splits_hint suggests for an M x N x K product
    on the current device (1: splitting does not help)."""
    return int(lib().nvfp4_gemm_splits_hint(M, N, K))


def gemm(a, b, out_dtype=torch.float32, out=None, stream=None, splits=None, workspace=None):
    """W4A4 product out [M][N] = ga * gb * sum_k a(m,k) b(n,k) (nvfp4_gemm):
    Y = X W^T for NVFP4 activations X [M][K] and weights W [N][K], both
    blocked along K.  a, b: dicts with "packed" ([rows][K/2] uint8),
    "scales" ([rows][K/16] uint8) and "gscale" (1-element float32), e.g. the
    results of quantize (AXIS_COLS) or quantize_residual.  Returns out, float32
    or bfloat16.
    splits: None (nvfp4_gemm), an int (nvfp4_gemm_splitk with that many
    ranges of K) or "auto" (the library's hint; nvfp4_gemm when it is 1).
    workspace: float32 device tensor of at least splits * M * N elements for
    the split product; allocated here when not given."""
    code = {torch.float32: OUT_F32, torch.bfloat16: OUT_BF16}[out_dtype]
    pa, pb = a["packed"], b["packed"]
    if pa.dim() != 2 or pb.dim() != 2 or pa.shape[1] != pb.shape[1]:
        raise ValueError("operands must be [rows][K/2] with the same K")
    M, N, K = pa.shape[0], pb.shape[0], pa.shape[1] * 2
    dev = pa.device
    pa = _need(pa, M * K // 2, torch.uint8, dev, "a['packed']")
    sa = _need(a["scales"], M * K // 16, torch.uint8, dev, "a['scales']")
    ga = _need(a["gscale"], 1, torch.float32, dev, "a['gscale']")
    pb = _need(pb, N * K // 2, torch.uint8, dev, "b['packed']")
    sb = _need(b["scales"], N * K // 16, torch.uint8, dev, "b['scales']")
    gb = _need(b["gscale"], 1, torch.float32, dev, "b['gscale']")
    out = _out({"out": out}, "out", (M, N), out_dtype, dev)
    if splits == "auto":
        splits = gemm_splits_hint(M, N, K)
        if splits <= 1:
            splits = None
    if splits is None:
        st = lib().nvfp4_gemm(_ptr(pa), _ptr(sa), _ptr(ga), _ptr(pb), _ptr(sb), _ptr(gb), M, N,
                              K, code, _ptr(out), _stream(stream))
        _check(st, "nvfp4_gemm")
        return out
    splits = int(splits)
    if workspace is None:
        workspace = torch.empty(max(1, splits) * M * N, dtype=torch.float32, device=dev)
    elif (not isinstance(workspace, torch.Tensor) or workspace.dtype != torch.float32
          or workspace.device != dev or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous float32 tensor on the operands' device")
    st = lib().nvfp4_gemm_splitk(_ptr(pa), _ptr(sa), _ptr(ga), _ptr(pb), _ptr(sb), _ptr(gb), M,
                                 N, K, splits, code, _ptr(out), _ptr(workspace),
                                 workspace.numel(), _stream(stream))
    _check(st, "nvfp4_gemm_splitk")
    return out


def gemm_splitk_noalloc(a, b, splits, out, stream=None):
    """The split product of gemm(a, b, splits=splits) through
    nvfp4_gemm_splitk_noalloc, whose per-range sums live in the library's
    fixed device scratch (at most NOALLOC_SCRATCH_FLOATS = splits * M * N):
    no workspace, and the call allocates nothing.  `out` ([M][N] float32 or
    bfloat16, preallocated) is written and returned.  Calls that overlap in
    time on one device race on the scratch."""
    pa, pb = a["packed"], b["packed"]
    if pa.dim() != 2 or pb.dim() != 2 or pa.shape[1] != pb.shape[1]:
        raise ValueError("operands must be [rows][K/2] with the same K")
    M, N, K = pa.shape[0], pb.shape[0], pa.shape[1] * 2
    dev = pa.device
    if not isinstance(out, torch.Tensor) or out.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out must be a preallocated float32 or bfloat16 tensor")
    code = OUT_F32 if out.dtype == torch.float32 else OUT_BF16
    pa = _need(pa, M * K // 2, torch.uint8, dev, "a['packed']")
    sa = _need(a["scales"], M * K // 16, torch.uint8, dev, "a['scales']")
    ga = _need(a["gscale"], 1, torch.float32, dev, "a['gscale']")
    pb = _need(pb, N * K // 2, torch.uint8, dev, "b['packed']")
    sb = _need(b["scales"], N * K // 16, torch.uint8, dev, "b['scales']")
    gb = _need(b["gscale"], 1, torch.float32, dev, "b['gscale']")
    out = _need(out, M * N, out.dtype, dev, "out")
    st = lib().nvfp4_gemm_splitk_noalloc(_ptr(pa), _ptr(sa), _ptr(ga), _ptr(pb), _ptr(sb),
                                         _ptr(gb), M, N, K, int(splits), code, _ptr(out),
                                         _stream(stream))
    _check(st, "nvfp4_gemm_splitk_noalloc")
    return out


def stream_pattern(x, packed, scales, stream=None):
    """The row quantizer's memory traffic without its arithmetic
    (nvfp4v_stream_pattern): reads x, writes packed and scales with the same
    sizes, launch shape and access order.  Measurement only; the bytes
    written are not NVFP4 codes."""
    x = _bf16_input(x)
    packed = _need(packed, x.numel() // 2, torch.uint8, x.device, "packed")
    scales = _need(scales, x.numel() // 16, torch.uint8, x.device, "scales")
    _check(lib().nvfp4v_stream_pattern(_ptr(x), x.numel() // 16, _ptr(packed), _ptr(scales),
                                       _stream(stream)), "nvfp4v_stream_pattern")
