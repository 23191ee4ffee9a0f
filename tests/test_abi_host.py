"""The C-ABI library on the host: it loads, it exports every symbol the
public headers declare, and it rejects bad arguments before any HIP call
(so these run without a GPU; the pointers below are never dereferenced)."""
import ctypes
import os
import re

import pytest

import nvfp4_block_scaled_wave64_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("nvfp4.h", "nvfp4_verify.h")]

A = ctypes.c_void_p(0x10000)  # aligned dummy device address (never touched)
B = ctypes.c_void_p(0x20000)
C = ctypes.c_void_p(0x30000)
MIS = ctypes.c_void_p(0x10002)


def declared_functions():
    names = []
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(nvfp4v?_[a-z_0-9]+)\s*\(",
                            text, flags=re.M)
    return names


def test_library_exports_every_declared_symbol():
    L = nv.lib()
    names = declared_functions()
    assert len(names) == 21, names
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(nv.SIGNATURES)


def test_status_strings():
    L = nv.lib()
    for s in range(8):
        assert L.nvfp4_status_string(s)
    assert b"alias" in L.nvfp4_status_string(6)
    assert b"scratch" in L.nvfp4_status_string(7)
    assert b"unknown" in L.nvfp4_status_string(99)


def q(**kw):
    """Status of nvfp4_quantize_ex for the given arguments; the timed variant
    must return the same status for them."""
    args = dict(in_=A, rows=32, cols=64, axis=nv.AXIS_COLS, mode=nv.MODE_4OVER6, rule=nv.RULE_MSE,
                flags=0, packed=B, scales=C, g=A, sel=None, err=None)
    args.update(kw)
    pos = (args["in_"], args["rows"], args["cols"], args["axis"], args["mode"], args["rule"],
           args["flags"], args["packed"], args["scales"], args["g"], args["sel"], args["err"])
    st = nv.lib().nvfp4_quantize_ex(*pos, None)
    assert nv.lib().nvfp4_quantize_ex_timed(*pos, A, B, None) == st
    return st


@pytest.mark.parametrize("kw,status", [
    (dict(in_=None), 1), (dict(packed=None), 1), (dict(scales=None), 1), (dict(g=None), 1),
    (dict(axis=2), 2), (dict(mode=3), 2), (dict(rule=-1), 2), (dict(rule=3), 2), (dict(flags=4), 2), (dict(flags=8), 2),
    (dict(rows=0), 3), (dict(cols=-16), 3), (dict(cols=40), 3),
    (dict(axis=nv.AXIS_ROWS, rows=24), 3), (dict(rows=1 << 40, cols=1 << 10), 3),
    (dict(in_=MIS), 4), (dict(sel=ctypes.c_void_p(0x10001)), 4),
    (dict(err=ctypes.c_void_p(0x10004)), 4), (dict(packed=ctypes.c_void_p(0x10002)), 4),
])
def test_quantize_rejects(kw, status):
    assert q(**kw) == status


def test_check_order_null_before_enum_before_shape_before_align():
    assert q(in_=None, mode=7, rows=0) == 1
    assert q(mode=7, rows=0, in_=MIS) == 2
    assert q(rows=0, in_=MIS) == 3


def test_other_entry_points_reject():
    L = nv.lib()
    assert L.nvfp4_amax(None, 16, A, None) == 1
    assert L.nvfp4_amax(A, 0, B, None) == 3
    assert L.nvfp4_amax(MIS, 16, B, None) == 4
    assert L.nvfp4_global_scale(A, 2, B, None) == 2
    assert L.nvfp4_global_scale(None, 0, B, None) == 1
    assert L.nvfp4_dequantize(A, B, C, 32, 64, nv.AXIS_COLS, 2, A, None) == 2
    assert L.nvfp4_dequantize(A, B, C, 32, 8, nv.AXIS_COLS, 0, A, None) == 3
    assert L.nvfp4_dequantize(A, B, C, 32, 64, nv.AXIS_COLS, 0, MIS, None) == 4
    assert L.nvfp4_quantize(None, 16, 16, 1, 0, 0, A, B, C, None) == 1
    assert L.nvfp4v_e2m1_encode_sweep(0xFFFFFFF0, 17, A, None) == 3
    assert L.nvfp4v_e2m1_encode_sweep(0, 0, A, None) == 3
    assert L.nvfp4v_e4m3_encode_sweep(0, 16, None, None) == 1
    assert L.nvfp4v_decode_tables(1.0, None, A, B, C, None) == 1
    assert L.nvfp4v_stream_pattern(None, 16, A, B, None) == 1
    assert L.nvfp4v_stream_pattern(A, 0, B, C, None) == 3
    assert L.nvfp4v_stream_pattern(MIS, 16, B, C, None) == 4


def dq(**kw):
    args = dict(in_=A, rows=32, cols=64, axis=nv.AXIS_COLS, mode=nv.MODE_4OVER6, rule=nv.RULE_MSE,
                flags=0, packed=B, scales=C, g=A, amax=B, sel=None, err=None)
    args.update(kw)
    return nv.lib().nvfp4_quantize_delayed(args["in_"], args["rows"], args["cols"], args["axis"],
                                           args["mode"], args["rule"], args["flags"],
                                           args["packed"], args["scales"], args["g"],
                                           args["amax"], args["sel"], args["err"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(g=None), 1), (dict(amax=None), 1), (dict(in_=None), 1), (dict(packed=None, flags=1), 1),
    (dict(flags=1), 2), (dict(flags=4), 2), (dict(rule=7), 2), (dict(rows=0), 3),
    (dict(amax=ctypes.c_void_p(0x20002)), 4), (dict(amax=A), 6),
])
def test_delayed_rejects(kw, status):
    """nvfp4_quantize_delayed: null, enum (GSCALE_GIVEN is implied, so only
    the accumulate flag is accepted), shape, alignment, and amax_out
    aliasing gscale_in."""
    assert dq(**kw) == status


def du(**kw):
    args = dict(in_=A, rows=32, cols=64, mode=nv.MODE_4OVER6, rule=nv.RULE_MSE, flags=0,
                pr=B, sr=C, pc=B, sc=C, g=A, selr=None, selc=None, errr=None, errc=None)
    args.update(kw)
    return nv.lib().nvfp4_quantize_dual(args["in_"], args["rows"], args["cols"], args["mode"],
                                        args["rule"], args["flags"], args["pr"], args["sr"],
                                        args["pc"], args["sc"], args["g"], args["selr"],
                                        args["selc"], args["errr"], args["errc"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(in_=None), 1), (dict(pc=None), 1), (dict(sr=None), 1), (dict(g=None), 1),
    (dict(selr=A), 1), (dict(errc=ctypes.c_void_p(0x40000)), 1),
    (dict(mode=2), 2), (dict(rule=3), 2), (dict(flags=4), 2),
    (dict(rows=24), 3), (dict(cols=40), 3), (dict(rows=0), 3),
    (dict(in_=MIS), 4), (dict(pc=ctypes.c_void_p(0x20002)), 4),
    (dict(selr=ctypes.c_void_p(0x10001), selc=A), 4),
])
def test_dual_rejects(kw, status):
    """nvfp4_quantize_dual: nulls (the bitmaps and the error sums come in
    pairs), enums, both extents multiples of 16, alignment."""
    assert du(**kw) == status


D = ctypes.c_void_p(0x40000)
E = ctypes.c_void_p(0x50000)


def co(**kw):
    args = dict(in_=A, rows=32, cols=64, flags=0, absmax=B, perm=C)
    args.update(kw)
    return nv.lib().nvfp4_channel_order(args["in_"], args["rows"], args["cols"], args["flags"],
                                        args["absmax"], args["perm"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(in_=None), 1), (dict(absmax=None), 1), (dict(perm=None), 1),
    (dict(flags=1), 2), (dict(flags=2), 2),
    (dict(rows=0), 3), (dict(cols=40), 3), (dict(cols=32784), 3),
    (dict(in_=MIS), 4), (dict(absmax=ctypes.c_void_p(0x20002)), 4),
    (dict(perm=ctypes.c_void_p(0x30001)), 4),
    (dict(absmax=ctypes.c_void_p(0x10100)), 6), (dict(perm=ctypes.c_void_p(0x200F0)), 6),
])
def test_channel_order_rejects(kw, status):
    """nvfp4_channel_order: nulls, flags (only the accumulate flag), shape
    (cols a multiple of 16 and at most 32768), alignment, and outputs that
    overlap the input or each other."""
    assert co(**kw) == status


def test_channel_order_accumulate_flag_passes_the_enum_check():
    # With the accumulate flag the first failing check is the shape's (a
    # call with every argument valid would launch, so none is made here).
    assert co(flags=4, rows=-1) == 3


def qr(**kw):
    args = dict(in_=A, rows=32, cols=64, perm=B, nres=16, mode=nv.MODE_4OVER6, rule=nv.RULE_MSE,
                flags=0, packed=C, scales=D, g=E)
    args.update(kw)
    return nv.lib().nvfp4_quantize_residual(args["in_"], args["rows"], args["cols"], args["perm"],
                                            args["nres"], args["mode"], args["rule"],
                                            args["flags"], args["packed"], args["scales"],
                                            args["g"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(in_=None), 1), (dict(perm=None), 1), (dict(packed=None), 1), (dict(scales=None), 1),
    (dict(g=None), 1),
    (dict(mode=2), 2), (dict(rule=3), 2), (dict(flags=2), 2), (dict(flags=4), 2),
    (dict(flags=16), 2),
    (dict(rows=0), 3), (dict(cols=40), 3), (dict(cols=32784), 3), (dict(nres=-16), 3),
    (dict(flags=8, rows=0), 3), (dict(flags=9, rows=0), 3),
    (dict(nres=8), 3), (dict(nres=80), 3),
    (dict(in_=MIS), 4), (dict(perm=ctypes.c_void_p(0x20002)), 4),
    (dict(packed=ctypes.c_void_p(0x30002)), 4), (dict(g=ctypes.c_void_p(0x50001)), 4),
    (dict(packed=ctypes.c_void_p(0x10800)), 6), (dict(scales=ctypes.c_void_p(0x200F0)), 6),
    (dict(g=ctypes.c_void_p(0x30100)), 6), (dict(scales=ctypes.c_void_p(0x30200)), 6),
])
def test_quantize_residual_rejects(kw, status):
    """nvfp4_quantize_residual: nulls, enums (GSCALE_GIVEN and
    RESIDUAL_DUPLICATE are the valid flags), shape (cols a multiple of 16 up to 32768, nres a multiple of 16
    in [0, cols]), alignment, and outputs overlapping the input, perm or
    each other."""
    assert qr(**kw) == status


F = ctypes.c_void_p(0x60000)


def rq(**kw):
    args = dict(in_=A, rows=32, cols=64, w=None, eps=1e-6, perm=B, nres=16, mode=nv.MODE_4OVER6,
                rule=nv.RULE_MSE, flags=0, packed=C, scales=D, g=E, amax=None)
    args.update(kw)
    return nv.lib().nvfp4_rmsnorm_quantize_residual(
        args["in_"], args["rows"], args["cols"], args["w"], args["eps"], args["perm"], args["nres"],
        args["mode"], args["rule"], args["flags"], args["packed"], args["scales"], args["g"],
        args["amax"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(in_=None), 1), (dict(perm=None), 1), (dict(packed=None), 1), (dict(g=None), 1),
    (dict(mode=5), 2), (dict(rule=4), 2), (dict(flags=2), 2), (dict(eps=-1.0), 2),
    (dict(eps=float("inf")), 2), (dict(eps=float("nan")), 2),
    (dict(cols=24592), 3), (dict(cols=40), 3), (dict(rows=0), 3), (dict(nres=24), 3),
    (dict(w=ctypes.c_void_p(0x60008)), 4), (dict(amax=ctypes.c_void_p(0x60002)), 4),
    (dict(in_=MIS), 4),
    (dict(amax=E), 6), (dict(w=ctypes.c_void_p(0x30000)), 6), (dict(g=ctypes.c_void_p(0x10010)), 6),
])
def test_rmsnorm_quantize_residual_rejects(kw, status):
    """nvfp4_rmsnorm_quantize_residual: nulls, enums (eps finite and >= 0,
    only GSCALE_GIVEN), shape (cols <= 24576), alignment (weight 16 bytes),
    outputs overlapping inputs or each other."""
    assert rq(**kw) == status


def test_binding_checks_caller_tensors():
    """The binding refuses a caller-supplied tensor of the wrong dtype,
    device, layout or size before any library call (CPU tensors stand in for
    device ones here)."""
    import torch
    cpu = torch.device("cpu")
    t = torch.zeros(8, dtype=torch.float32)
    assert nv._need(t, 8, torch.float32, cpu, "t") is t
    with pytest.raises(ValueError):
        nv._need(t, 9, torch.float32, cpu, "t")
    with pytest.raises(TypeError):
        nv._need(t, 8, torch.int32, cpu, "t")
    with pytest.raises(TypeError):
        nv._need(torch.zeros(4, 4)[:, ::2], 8, torch.float32, cpu, "t")
    with pytest.raises(TypeError):
        nv._need(t.numpy(), 8, torch.float32, cpu, "t")
    assert nv._out({}, "k", (3, 5), torch.uint8, cpu).shape == (3, 5)
    with pytest.raises(ValueError):
        nv._out({"k": torch.zeros(14, dtype=torch.uint8)}, "k", (3, 5), torch.uint8, cpu)
    with pytest.raises(ValueError):
        nv.quantize(torch.zeros(16, 16, dtype=torch.bfloat16))  # host memory


G = ctypes.c_void_p(0x70000)


def gm(**kw):
    args = dict(pa=A, sa=B, ga=C, pb=D, sb=E, gb=F, m=32, n=32, k=64, dtype=nv.OUT_F32, out=G)
    args.update(kw)
    return nv.lib().nvfp4_gemm(args["pa"], args["sa"], args["ga"], args["pb"], args["sb"],
                               args["gb"], args["m"], args["n"], args["k"], args["dtype"],
                               args["out"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(pa=None), 1), (dict(sa=None), 1), (dict(ga=None), 1), (dict(pb=None), 1),
    (dict(sb=None), 1), (dict(gb=None), 1), (dict(out=None), 1),
    (dict(dtype=2), 2), (dict(dtype=-1), 2),
    (dict(m=0), 3), (dict(n=-4), 3), (dict(k=0), 3), (dict(k=40), 3),
    (dict(k=(1 << 24) + 16), 3), (dict(m=1 << 40, n=1 << 10), 3), (dict(m=1 << 31, k=1 << 16), 3),
    (dict(n=(1 << 24) + 1, m=1), 3),
    (dict(pa=ctypes.c_void_p(0x10002)), 4), (dict(pb=ctypes.c_void_p(0x40001)), 4),
    (dict(ga=ctypes.c_void_p(0x30002)), 4), (dict(out=ctypes.c_void_p(0x70002)), 4),
    (dict(out=ctypes.c_void_p(0x70001), dtype=nv.OUT_BF16), 4),
    (dict(out=A), 6), (dict(out=ctypes.c_void_p(0x10200)), 6),
    (dict(out=ctypes.c_void_p(0x5FFF0)), 6), (dict(out=ctypes.c_void_p(0x4FF00)), 6),
])
def test_gemm_rejects(kw, status):
    """nvfp4_gemm: nulls, out_dtype, shape (positive extents, k a multiple of
    16 up to 2^24, n up to 2^24, products of extents up to 2^46), alignment (codes and
    scalars 4 bytes, out its element size) and an output overlapping any
    input."""
    assert gm(**kw) == status


W = ctypes.c_void_p(0x90000)


def gs(**kw):
    args = dict(pa=A, sa=B, ga=C, pb=D, sb=E, gb=F, m=32, n=32, k=256, splits=2,
                dtype=nv.OUT_F32, out=G, ws=W, nws=2048)
    args.update(kw)
    return nv.lib().nvfp4_gemm_splitk(args["pa"], args["sa"], args["ga"], args["pb"], args["sb"],
                                      args["gb"], args["m"], args["n"], args["k"], args["splits"],
                                      args["dtype"], args["out"], args["ws"], args["nws"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(ws=None), 1), (dict(pa=None), 1), (dict(out=None), 1),
    (dict(dtype=3), 2),
    (dict(m=0), 3), (dict(k=40), 3), (dict(splits=0), 3), (dict(splits=-1), 3),
    (dict(splits=3), 3), (dict(splits=65, k=64 * 128), 3), (dict(nws=2047), 3),
    (dict(k=64, splits=2, nws=1 << 20), 3),
    (dict(ws=ctypes.c_void_p(0x90002)), 4), (dict(out=ctypes.c_void_p(0x70002)), 4),
    (dict(ws=ctypes.c_void_p(0x70800)), 6), (dict(ws=ctypes.c_void_p(0x6FF00)), 6),
    (dict(ws=ctypes.c_void_p(0x10400)), 6), (dict(ws=ctypes.c_void_p(0x3FFF8), nws=4096), 6),
    (dict(out=D), 6),
])
def test_gemm_splitk_rejects(kw, status):
    """nvfp4_gemm_splitk: nvfp4_gemm's checks plus a workspace that is null,
    too small (fewer than splits * m * n floats), not 4-byte aligned or
    overlapping an input or the output, and a split count outside
    1 .. min(64, ceil(k / 128))."""
    assert gs(**kw) == status


def test_gemm_splits_hint_rejects_bad_shapes():
    """The hint returns 0, before any HIP call, for shapes nvfp4_gemm rejects."""
    L = nv.lib()
    assert L.nvfp4_gemm_splits_hint(0, 16, 16) == 0
    assert L.nvfp4_gemm_splits_hint(16, 16, 40) == 0
    assert L.nvfp4_gemm_splits_hint(16, (1 << 24) + 1, 16) == 0


FAR = {name: ctypes.c_void_p((i + 1) << 32)
       for i, name in enumerate(("pa", "sa", "ga", "pb", "sb", "gb", "out"))}


def gn(**kw):
    args = dict(pa=A, sa=B, ga=C, pb=D, sb=E, gb=F, m=32, n=32, k=256, splits=2,
                dtype=nv.OUT_F32, out=G)
    args.update(kw)
    return nv.lib().nvfp4_gemm_splitk_noalloc(args["pa"], args["sa"], args["ga"], args["pb"],
                                              args["sb"], args["gb"], args["m"], args["n"],
                                              args["k"], args["splits"], args["dtype"],
                                              args["out"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(pa=None), 1), (dict(gb=None), 1), (dict(out=None), 1),
    (dict(dtype=3), 2),
    (dict(m=0), 3), (dict(k=40), 3), (dict(splits=0), 3), (dict(splits=3), 3),
    (dict(splits=65, k=64 * 128), 3),
    (dict(out=ctypes.c_void_p(0x70002)), 4), (dict(pb=ctypes.c_void_p(0x40001)), 4),
    (dict(out=D), 6), (dict(out=A), 6),
    # splits * m * n above the fixed scratch of 2^23 floats, checked before any
    # HIP call (operands placed 4 GiB apart so that they do not overlap)
    (dict(FAR, m=4097, n=1024, k=1024, splits=2), 7),
    (dict(FAR, m=1, n=1 << 22, k=512, splits=3), 7),
])
def test_gemm_splitk_noalloc_rejects(kw, status):
    """nvfp4_gemm_splitk_noalloc: nvfp4_gemm_splitk's checks without the
    workspace ones, plus the scratch limit (NVFP4_ERR_SCRATCH when
    splits * m * n > 2^23), all before any HIP call."""
    assert gn(**kw) == status


def P(gib, off=0):
    """A fake device address `gib` GiB up (plus off bytes), never touched."""
    return ctypes.c_void_p((gib << 30) + off)


# 32 x 64 tensor: input 4096 B, codes 1024 B, scales 128 B, bitmap 16 B.
QX = dict(in_=P(1), packed=P(2), scales=P(3), g=P(4), sel=P(5), err=P(6))


@pytest.mark.parametrize("kw", [
    dict(packed=P(1, 4092)), dict(scales=P(1)), dict(g=P(1, 100)), dict(sel=P(1, 4080)),
    dict(err=P(1, 8)), dict(scales=P(2, 1020)), dict(g=P(3, 124)), dict(sel=P(2)),
    dict(err=P(4)), dict(err=P(5, 8)),
])
def test_quantize_rejects_overlapping_outputs(kw):
    """nvfp4_quantize_ex: no output (codes, scales, g, bitmap, error sum) may
    overlap the input or another output."""
    args = dict(QX)
    args.update(kw)
    assert q(**args) == 6


def test_quantize_accepts_adjacent_outputs():
    """Ranges that only touch are not overlaps: the checks stop at the HIP
    launch, which a host without a GPU reports as a launch failure, not an
    aliasing error."""
    assert q(**dict(QX, packed=P(1, 4096), scales=P(1, 4096 + 1024))) not in (1, 2, 3, 4, 6)


@pytest.mark.parametrize("kw", [
    dict(pr=P(1, 100)), dict(pc=P(2, 1000)), dict(sc=P(3, 64)), dict(g=P(5)),
    dict(selc=P(5, 8)), dict(errr=P(10)), dict(errc=P(4)),
])
def test_dual_rejects_overlapping_outputs(kw):
    args = dict(in_=P(1), pr=P(2), sr=P(3), pc=P(4), sc=P(5), g=P(6), selr=P(7), selc=P(8),
                errr=P(9), errc=P(10))
    args.update(kw)
    assert du(**args) == 6


@pytest.mark.parametrize("out,dtype,g", [(P(1, 992), 0, P(3)), (P(2, 64), 1, P(3)),
                                         (P(3), 0, P(3)), (P(4), 0, P(4, 8188)),
                                         (P(4), 1, P(4, 4092))])
def test_dequantize_rejects_overlap(out, dtype, g):
    """out (32 x 64: fp32 8192 B, bf16 4096 B) may not overlap the codes
    (1 GiB up, 1024 B), scales (2 GiB up, 128 B) or g it reads."""
    L = nv.lib()
    assert L.nvfp4_dequantize(P(1), P(2), g, 32, 64, nv.AXIS_COLS, dtype, out, None) == 6


def test_check_order_rejects():
    L = nv.lib()
    assert L.nvfp4_check_order(None, 16, A, None) == 1
    assert L.nvfp4_check_order(A, 16, None, None) == 1
    assert L.nvfp4_check_order(A, 0, B, None) == 3
    assert L.nvfp4_check_order(A, 32769, B, None) == 3
    assert L.nvfp4_check_order(MIS, 16, B, None) == 4
    assert L.nvfp4_check_order(A, 16, ctypes.c_void_p(0x10002), None) == 4
    assert L.nvfp4_check_order(A, 16, ctypes.c_void_p(0x10000 + 60), None) == 6
