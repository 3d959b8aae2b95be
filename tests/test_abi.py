"""The C-ABI library loads, exports every entry point include/nvfp4.h
declares, and rejects invalid arguments before any HIP call (CPU only: no
call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest
import torch

import bit_linear_layer_amd as nv

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "nvfp4.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(nvfp4_[a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_declares_the_expected_api():
    fns = declared_functions()
    for f in ("nvfp4_quantize", "nvfp4_quantize_workspace_bytes", "nvfp4_gemm",
              "nvfp4_gemm_fused_segments", "nvfp4_silu_mul", "nvfp4_status_string", "nvfp4_version"):
        assert f in fns


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(nv.lib_path)
    for f in declared_functions():
        assert hasattr(lib, f), f


def test_version_and_status_strings():
    assert nv.nvfp4_version() >= 100
    assert nv.nvfp4_status_string(0) == "ok"
    for code in range(-1, -12, -1):
        assert nv.nvfp4_status_string(code) not in ("", "unknown status")


def test_workspace_bytes():
    assert nv.nvfp4_quantize_workspace_bytes(1, 16) == 4
    assert 4 <= nv.nvfp4_quantize_workspace_bytes(32768, 5120) <= 4096


FAKE = 1 << 20  # a well-aligned non-null pointer value; never dereferenced on these paths


def q(**kw):
    args = dict(x=FAKE, dt=0, rows=4, cols=32, ldx=32, codes=FAKE, ldc=16, scales=FAKE, lds=8,
                g=FAKE, flags=0, ws=FAKE, wsb=4096, stream=None)
    args.update(kw)
    return nv.load().nvfp4_quantize(args["x"], args["dt"], args["rows"], args["cols"], args["ldx"],
                                    args["codes"], args["ldc"], args["scales"], args["lds"], args["g"],
                                    args["flags"], args["ws"], args["wsb"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), -1), (dict(codes=None), -1), (dict(g=None), -1),
    (dict(dt=7), -3), (dict(flags=9), -9),
    (dict(cols=24, ldx=24), -2), (dict(rows=0), -2), (dict(rows=-3), -2),
    (dict(ldx=16), -4), (dict(ldc=8), -4), (dict(lds=1), -4),
    (dict(x=FAKE + 2), -5), (dict(ws=None), -8), (dict(wsb=0), -8),
    (dict(rows=1 << 31), -11),
])
def test_quantize_rejects_bad_arguments(kw, status):
    assert q(**kw) == status


def tensor(rows=4, cols=32, ldc=16, lds=8, codes=FAKE, scales=FAKE, g=FAKE):
    return nv._Tensor(codes, scales, g, rows, cols, ldc, lds)


def gemm(a=None, w=None, out=FAKE, dt=0, ld=8):
    a = a or tensor()
    w = w or tensor(rows=8)
    return nv.load().nvfp4_gemm(ctypes.byref(a), ctypes.byref(w), out, dt, ld, None)


@pytest.mark.parametrize("kw,status", [
    (dict(a=tensor(codes=0)), -1), (dict(w=tensor(rows=8, g=0)), -1), (dict(out=None), -1),
    (dict(a=tensor(cols=48, ldc=32)), -2), (dict(a=tensor(cols=20)), -2),
    (dict(dt=5), -3), (dict(ld=4), -4), (dict(a=tensor(ldc=24)), -4), (dict(a=tensor(lds=4)), -4),
    (dict(a=tensor(codes=FAKE + 8)), -5), (dict(out=FAKE + 1), -5),
    # operands of 2^31 code bytes or more: beyond the kernels' 32-bit offsets
    (dict(w=tensor(rows=1 << 20, ldc=1 << 11)), -11), (dict(a=tensor(rows=1 << 27, lds=16)), -11),
])
def test_gemm_rejects_bad_arguments(kw, status):
    assert gemm(**kw) == status


def fused(nseg=2, offs=(0, 4, 8), gate=None, sg=FAKE):
    a, w = tensor(), tensor(rows=8)
    arr = (ctypes.c_int64 * len(offs))(*offs)
    return nv.load().nvfp4_gemm_fused_segments(ctypes.byref(a), ctypes.byref(w), nseg, arr, sg,
                                               None if gate is None else ctypes.byref(gate), FAKE, 0, 8, None)


@pytest.mark.parametrize("kw,status", [
    (dict(nseg=0, offs=(0,)), -6), (dict(nseg=17, offs=tuple(range(18))), -6),
    (dict(offs=(0, 4, 7)), -6), (dict(offs=(1, 4, 8)), -6), (dict(offs=(0, 9, 8)), -6),
    (dict(sg=None), -1),
    (dict(gate=nv._Gate(2, -1, None, None)), -7), (dict(gate=nv._Gate(0, 0, FAKE, FAKE)), -7),
    (dict(gate=nv._Gate(0, 1, None, FAKE)), -7),
])
def test_fused_rejects_bad_arguments(kw, status):
    assert fused(**kw) == status


def test_silu_mul_rejects_bad_arguments():
    f = nv.load().nvfp4_silu_mul
    assert f(None, 4, 16, 32, FAKE, 16, None, 0, None) == -1
    assert f(FAKE, 4, 12, 32, FAKE, 16, None, 0, None) == -2
    assert f(FAKE, 4, 16, 24, FAKE, 16, None, 0, None) == -4
    assert f(FAKE + 4, 4, 16, 32, FAKE, 16, None, 0, None) == -5
    assert f(FAKE, 4, 16, 32, FAKE, 16, FAKE, 0, None) == -8
    assert f(FAKE, 4, 8, 16, FAKE, 8, FAKE, 4096, None) == -2  # amax partials need inter % 16 == 0


def swiglu(a=None, w=None, sg=FAKE, h=FAKE, ldh=16, ws=None, wsb=0, hq=None):
    a = a or tensor()
    w = w or tensor(rows=32)  # inter = 16
    return nv.load().nvfp4_gemm_swiglu(ctypes.byref(a), ctypes.byref(w), sg, h, ldh, ws, wsb,
                                       None if hq is None else ctypes.byref(hq), None)


@pytest.mark.parametrize("kw,status", [
    (dict(sg=None), -1), (dict(h=None), -1), (dict(a=tensor(g=0)), -1),
    (dict(w=tensor(rows=31)), -2), (dict(w=tensor(rows=24)), -2),  # odd rows; inter % 16 != 0
    (dict(w=tensor(rows=32, cols=48, ldc=32)), -2),
    (dict(ldh=8), -4), (dict(ldh=20), -4), (dict(h=FAKE + 2), -5),
    (dict(ws=FAKE, wsb=0), -8),
    (dict(h=None, hq=tensor(rows=4, cols=32, g=0)), -1), (dict(h=None, hq=tensor(rows=5, cols=16)), -2),
    (dict(h=None, hq=tensor(rows=4, cols=16, ldc=4)), -4),
])
def test_swiglu_rejects_bad_arguments(kw, status):
    assert swiglu(**kw) == status


def test_kv_fp8_entry_points_reject_bad_arguments():
    lib = nv.load()
    cal = lib.nvfp4_kv_fp8_calibrate
    assert cal(None, 0, 4, 32, 32, FAKE, FAKE, 4096, None) == -1
    assert cal(FAKE, 0, 4, 32, 32, FAKE, None, 4096, None) == -1
    assert cal(FAKE, 3, 4, 32, 32, FAKE, FAKE, 4096, None) == -3
    assert cal(FAKE, 0, 4, 24, 24, FAKE, FAKE, 4096, None) == -2
    assert cal(FAKE, 0, 4, 32, 36, FAKE, FAKE, 4096, None) == -4
    assert cal(FAKE, 0, 4, 32, 32, FAKE, FAKE, 0, None) == -8
    qz = lib.nvfp4_kv_fp8_quantize
    assert qz(FAKE, 0, 4, 32, 32, None, 4, None, 32, FAKE, None) == -1
    assert qz(FAKE, 0, 4, 32, 32, None, 3, FAKE, 32, FAKE, None) == -2  # too few cache rows without slots
    assert qz(FAKE, 0, 4, 32, 32, None, 4, FAKE, 36, FAKE, None) == -4
    assert qz(FAKE, 0, 4, 32, 32, None, 4, FAKE, 16, FAKE, None) == -4
    assert qz(FAKE, 0, 4, 32, 32, FAKE + 4, 4, FAKE, 32, FAKE, None) == -5
    assert qz(FAKE + 8, 0, 4, 32, 32, None, 4, FAKE, 32, FAKE, None) == -5
    assert qz(FAKE, 0, 4, 32, 32, None, 1 << 31, FAKE, 32, FAKE, None) == -11
    dq = lib.nvfp4_kv_fp8_dequantize
    assert dq(FAKE, 4, 32, 32, None, FAKE, 0, 32, None) == -1
    assert dq(FAKE, 4, 32, 32, FAKE, FAKE, 2, 32, None) == -3
    assert dq(FAKE, 4, 40, 40, FAKE, FAKE, 0, 40, None) == -2
    assert dq(FAKE, 4, 32, 32, FAKE, FAKE, 1, 34, None) == -4
    assert dq(FAKE, 4, 32, 32, FAKE, FAKE + 8, 0, 32, None) == -5


def test_harmonize_rejects_bad_arguments():
    f = nv.load().nvfp4_harmonize_scales

    def call(w=None, n=2, offs=(0, 4, 8), sg=FAKE, out=FAKE, ld=8, g=FAKE):
        w = w or tensor(rows=8)
        arr = (ctypes.c_int64 * len(offs))(*offs)
        return f(ctypes.byref(w), n, arr, sg, out, ld, g, None)
    assert call(sg=None) == -1 and call(out=None) == -1 and call(g=None) == -1
    assert call(w=tensor(rows=8, scales=0)) == -1
    assert call(w=tensor(rows=8, cols=24)) == -2
    assert call(ld=1) == -4
    assert call(g=FAKE + 2) == -5
    assert call(n=0, offs=(0,)) == -6 and call(offs=(0, 4, 7)) == -6 and call(offs=(0, 9, 8)) == -6


def qn(**kw):
    args = dict(x=FAKE, dt=0, rows=4, cols=32, ldx=32, codes=FAKE, ldc=16, scales=FAKE, lds=8,
                g=FAKE, flags=0, stream=None)
    args.update(kw)
    return nv.load().nvfp4_quantize_noalloc(args["x"], args["dt"], args["rows"], args["cols"], args["ldx"],
                                            args["codes"], args["ldc"], args["scales"], args["lds"], args["g"],
                                            args["flags"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), -1), (dict(g=None), -1), (dict(dt=7), -3), (dict(flags=9), -9), (dict(flags=2), -9),
    (dict(cols=24, ldx=24), -2), (dict(rows=0), -2), (dict(ldx=16), -4), (dict(x=FAKE + 2), -5),
    (dict(rows=1 << 31), -11),
])
def test_quantize_noalloc_rejects_bad_arguments(kw, status):
    assert qn(**kw) == status


def test_decode_weight_bytes():
    # 2176 groups x 8 K slices x (5 chunks x 1152 bytes): exactly the codes
    # and scales of a 34816 x 5120 weight
    assert nv.nvfp4_decode_weight_bytes(34816, 5120) == 34816 * 5120 // 2 + 34816 * 5120 // 16
    assert nv.nvfp4_decode_weight_bytes(1, 16) == 8 * 1152
    assert nv.nvfp4_decode_weight_bytes(1, 8208) == 0
    assert nv.nvfp4_decode_weight_bytes(1, 24) == 0
    assert nv.nvfp4_decode_weight_bytes(0, 16) == 0


def gemm_decode(a=None, w=None, n_seg=1, offs=None, out=FAKE, dt=0, ld=8, gate=None):
    a = a or tensor()
    w = w or nv._DecodeWeight(FAKE, 8, 32)
    offs = offs or [0, w.rows]
    arr = (ctypes.c_int64 * len(offs))(*offs)
    return nv.load().nvfp4_gemm_decode(ctypes.byref(a), ctypes.byref(w), n_seg, arr, FAKE,
                                       None if gate is None else ctypes.byref(gate), out, dt, ld, None)


@pytest.mark.parametrize("kw,status", [
    (dict(a=tensor(rows=17)), -2), (dict(a=tensor(cols=48, ldc=32, lds=8)), -2),
    (dict(w=nv._DecodeWeight(None, 8, 32)), -1), (dict(w=nv._DecodeWeight(FAKE + 8, 8, 32)), -5),
    (dict(w=nv._DecodeWeight(FAKE, 8, 8208)), -2), (dict(out=None), -1), (dict(ld=4), -4),
    (dict(offs=[0, 4]), -6), (dict(n_seg=0), -6), (dict(dt=5), -3),
    (dict(gate=nv._Gate(0, 0, FAKE, FAKE)), -7),
])
def test_gemm_decode_rejects_bad_arguments(kw, status):
    assert gemm_decode(**kw) == status


def linear_decode(x=FAKE, dt=0, rows=8, ldx=32, w=None, out=FAKE, ld=8):
    w = w or nv._DecodeWeight(FAKE, 8, 32)
    arr = (ctypes.c_int64 * 2)(0, w.rows)
    return nv.load().nvfp4_linear_decode(x, dt, rows, ldx, None, ctypes.byref(w), 1, arr, FAKE, None, out, 0,
                                         ld, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), -1), (dict(rows=17), -2), (dict(rows=0), -2), (dict(dt=3), -3),
    (dict(ldx=24), -4), (dict(ldx=36), -4), (dict(x=FAKE + 2), -5), (dict(out=None), -1),
])
def test_linear_decode_rejects_bad_arguments(kw, status):
    assert linear_decode(**kw) == status


def cpu_nvfp4(rows, cols):
    ldc = max(16, (cols // 2 + 15) // 16 * 16)
    lds = max(16, (cols // 16 + 15) // 16 * 16)
    return nv.NVFP4Tensor(torch.zeros((rows, ldc), dtype=torch.uint8), torch.zeros((rows, lds), dtype=torch.uint8),
                          torch.zeros(1), rows, cols)


@pytest.mark.parametrize("out", [torch.zeros((4, 7)), torch.zeros((5, 8)), torch.zeros((8, 4)).t(),
                                 torch.zeros((4, 8), dtype=torch.float64)])
def test_binding_rejects_bad_outputs(out):
    """The binding checks caller-supplied outputs before calling the library:
    wrong shape, non-contiguous rows, or (here, on the CPU) a host tensor."""
    a, w = cpu_nvfp4(4, 32), cpu_nvfp4(8, 32)
    with pytest.raises(nv.NVFP4Error):
        nv.nvfp4_gemm(a, w, out)
    with pytest.raises(nv.NVFP4Error):
        nv.nvfp4_gemm_fused_segments(a, w, [0, 8], torch.zeros(1), out)


def test_binding_rejects_mismatched_quantize_target():
    x = torch.zeros((4, 32), dtype=torch.bfloat16)
    for q in (cpu_nvfp4(5, 32), cpu_nvfp4(4, 48), cpu_nvfp4(4, 32)):
        with pytest.raises(nv.NVFP4Error):
            nv.nvfp4_quantize(x, q, nv.SCALE_DYNAMIC, torch.zeros(1))
    with pytest.raises(nv.NVFP4Error):
        nv.nvfp4_quantize(torch.zeros((4, 32)).t(), cpu_nvfp4(32, 4))
