"""Drive every C entry point of a libnvfp4 built from api.hip as host C++
under AddressSanitizer + UBSan with stub launchers (tests/sanitize/
stub_launchers.cpp): valid calls that reach a launcher, and each rejection
path.  Run in a process that preloads the sanitizer runtime; any report
aborts it.  Usage: python abi_driver.py LIB"""
import ctypes
import sys

P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
FAKE = 1 << 20  # aligned fake device address: never dereferenced by the host layer


class Tensor(ctypes.Structure):
    _fields_ = [("codes", P), ("scales", P), ("global_scale", P), ("rows", I64), ("cols", I64),
                ("ld_codes", I64), ("ld_scales", I64)]


class Gate(ctypes.Structure):
    _fields_ = [("b_segment", I32), ("a_segment", I32), ("A_log", P), ("dt_bias", P)]


class Gdn(ctypes.Structure):
    _fields_ = [("q", P), ("ld_q", I64), ("k", P), ("ld_k", I64), ("v", P), ("ld_v", I64), ("beta", P),
                ("ld_beta", I64), ("g", P), ("ld_g", I64)]


class DecodeWeight(ctypes.Structure):
    _fields_ = [("data", P), ("rows", I64), ("cols", I64)]


_libc = ctypes.CDLL(None)
_libc.malloc.restype = P
_libc.malloc.argtypes = [ctypes.c_size_t]
_kept = []


def offsets(*v):
    """A host int64 array in its own malloc'ed block of exactly len(v)
    elements, so the sanitizer sees a read past its end (ctypes' own arrays
    live inside the interpreter's pools, without redzones)."""
    arr = (I64 * len(v))(*v)
    ptr = _libc.malloc(ctypes.sizeof(arr))
    ctypes.memmove(ptr, arr, ctypes.sizeof(arr))
    _kept.append(ptr)
    return ptr


def main(path):
    L = ctypes.CDLL(path)
    L.nvfp4_status_string.restype = ctypes.c_char_p
    L.nvfp4_quantize_workspace_bytes.restype = ctypes.c_size_t
    L.nvfp4_quantize_workspace_bytes.argtypes = [I64, I64]
    L.nvfp4_gdn_workspace_bytes.restype = ctypes.c_size_t
    L.nvfp4_gdn_workspace_bytes.argtypes = [I64, I32]
    L.nvfp4_decode_weight_bytes.restype = ctypes.c_size_t
    L.nvfp4_decode_weight_bytes.argtypes = [I64, I64]
    checks = 0

    def expect(got, want, what):
        nonlocal checks
        checks += 1
        if got != want:
            raise SystemExit(f"{what}: got {got}, want {want}")

    # quantize
    q = L.nvfp4_quantize
    q.argtypes = [P, I32, I64, I64, I64, P, I64, P, I64, P, I32, P, ctypes.c_size_t, P]
    for rows, cols in ((1, 16), (64, 256), (65, 256), (4096, 5120), (1, 1 << 20)):
        ws = L.nvfp4_quantize_workspace_bytes(rows, cols)
        for flags in (0, 1, 2):
            expect(q(FAKE, 0, rows, cols, cols, FAKE, cols // 2, FAKE, cols // 16, FAKE, flags, FAKE, ws, None), 0,
                   f"quantize {rows}x{cols} flags {flags}")
        expect(q(FAKE, 0, rows, cols, cols, FAKE, cols // 2, FAKE, cols // 16, FAKE, 0, FAKE, ws - 4, None), -8,
               "short workspace")
    for bad, st in ((dict(x=None), -1), (dict(dt=9), -3), (dict(flags=7), -9), (dict(cols=24), -2),
                    (dict(rows=1 << 31), -11), (dict(ldx=8), -4), (dict(x=FAKE + 4), -5)):
        a = dict(x=FAKE, dt=0, rows=4, cols=32, ldx=32, flags=0)
        a.update(bad)
        expect(q(a["x"], a["dt"], a["rows"], a["cols"], a["ldx"], FAKE, 16, FAKE, 8, FAKE, a["flags"], FAKE, 4096,
                 None), st, f"quantize {bad}")
    for rows in (0, -1, 1, 7, 1 << 40):
        for cols in (0, 15, 16, 1 << 20):
            L.nvfp4_quantize_workspace_bytes(rows, cols)

    # GEMMs
    a = Tensor(FAKE, FAKE, FAKE, 8, 256, 128, 16)
    w = Tensor(FAKE, FAKE, FAKE, 96, 256, 128, 16)
    L.nvfp4_gemm.argtypes = [ctypes.POINTER(Tensor), ctypes.POINTER(Tensor), P, I32, I64, P]
    expect(L.nvfp4_gemm(ctypes.byref(a), ctypes.byref(w), FAKE, 0, 96, None), 0, "gemm")
    fs = L.nvfp4_gemm_fused_segments
    fs.argtypes = [ctypes.POINTER(Tensor), ctypes.POINTER(Tensor), I32, P, P, ctypes.POINTER(Gate), P, I32, I64, P]
    for n in range(1, 17):
        offs = offsets(*[96 * i // n for i in range(n)], 96)
        gate = Gate(n - 2, n - 1, FAKE, FAKE) if n >= 2 else None
        expect(fs(ctypes.byref(a), ctypes.byref(w), n, offs, FAKE, None if gate is None else ctypes.byref(gate),
                  FAKE, 1, 96, None), 0 if all(96 * i // n < 96 * (i + 1) // n for i in range(n)) else -6,
               f"fused {n} segments")
    expect(fs(ctypes.byref(a), ctypes.byref(w), 17, offsets(*range(0, 96, 6), 90, 96), FAKE, None, FAKE, 0, 96, None),
           -6, "17 segments")
    expect(fs(ctypes.byref(a), ctypes.byref(w), 2, offsets(0, 0, 96), FAKE, None, FAKE, 0, 96, None), -6, "empty seg")
    expect(fs(ctypes.byref(a), ctypes.byref(w), 2, offsets(0, 48, 96), FAKE, ctypes.byref(Gate(1, 1, FAKE, FAKE)),
              FAKE, 0, 96, None), -7, "gate b == a")
    expect(fs(ctypes.byref(a), ctypes.byref(w), 2, offsets(0, 48, 96), FAKE, ctypes.byref(Gate(0, 1, None, None)),
              FAKE, 0, 96, None), -7, "gate without A_log")
    # a launcher failure is reported with the HIP text
    L.nvfp4_stub_set_launch_status(1)
    expect(L.nvfp4_gemm(ctypes.byref(a), ctypes.byref(w), FAKE, 0, 96, None), -10, "launch failure")
    if b"HIP error" not in L.nvfp4_status_string(-10):
        raise SystemExit("status text of a HIP error")
    L.nvfp4_stub_set_launch_status(0)

    sw = L.nvfp4_gemm_swiglu
    sw.argtypes = [ctypes.POINTER(Tensor), ctypes.POINTER(Tensor), P, P, I64, P, ctypes.c_size_t,
                   ctypes.POINTER(Tensor), P]
    hq = Tensor(FAKE, FAKE, FAKE, 8, 48, 32, 16)
    expect(sw(ctypes.byref(a), ctypes.byref(w), FAKE, FAKE, 48, FAKE, 4096, ctypes.byref(hq), None), 0, "swiglu")
    expect(sw(ctypes.byref(a), ctypes.byref(w), FAKE, None, 0, None, 0, None, None), -1, "swiglu no output")

    L.nvfp4_silu_mul.argtypes = [P, I64, I64, I64, P, I64, P, ctypes.c_size_t, P]
    expect(L.nvfp4_silu_mul(FAKE, 8, 64, 128, FAKE, 64, FAKE, 4096, None), 0, "silu_mul")

    # KV cache, harmonization
    L.nvfp4_kv_fp8_calibrate.argtypes = [P, I32, I64, I64, I64, P, P, ctypes.c_size_t, P]
    expect(L.nvfp4_kv_fp8_calibrate(FAKE, 0, 64, 128, 128, FAKE, FAKE, 4096, None), 0, "kv calibrate")
    L.nvfp4_kv_fp8_quantize.argtypes = [P, I32, I64, I64, I64, P, I64, P, I64, P, P]
    expect(L.nvfp4_kv_fp8_quantize(FAKE, 0, 64, 128, 128, FAKE, 100, FAKE, 128, FAKE, None), 0, "kv write")
    expect(L.nvfp4_kv_fp8_quantize(FAKE, 0, 64, 128, 128, None, 10, FAKE, 128, FAKE, None), -2, "kv short cache")
    L.nvfp4_kv_fp8_dequantize.argtypes = [P, I64, I64, I64, P, P, I32, I64, P]
    expect(L.nvfp4_kv_fp8_dequantize(FAKE, 64, 128, 128, FAKE, FAKE, 0, 128, None), 0, "kv read")
    hz = L.nvfp4_harmonize_scales
    hz.argtypes = [ctypes.POINTER(Tensor), I32, P, P, P, I64, P, P]
    expect(hz(ctypes.byref(w), 16, offsets(*range(0, 96, 6), 96), FAKE, FAKE, 16, FAKE, None), 0, "harmonize 16")
    expect(hz(ctypes.byref(w), 2, offsets(0, 50, 40), FAKE, FAKE, 16, FAKE, None), -6, "harmonize bad table")

    # gated delta rule
    ws = L.nvfp4_gdn_workspace_bytes(100, 4)
    g = Gdn(FAKE, 256, FAKE, 256, FAKE, 512, FAKE, 4, FAKE, 4)
    gd = L.nvfp4_gdn_recurrence
    gd.argtypes = [ctypes.POINTER(Gdn), I32, I64, I32, I32, I32, P, P, P, I32, I64, P, ctypes.c_size_t, P]
    expect(gd(ctypes.byref(g), 1, 100, 2, 4, 1, None, None, FAKE, 1, 512, FAKE, ws, None), 0, "gdn")
    expect(gd(ctypes.byref(g), 1, 100, 2, 4, 1, None, None, FAKE, 1, 512, FAKE, ws - 1, None), -8, "gdn workspace")
    expect(gd(ctypes.byref(g), 1, 100, 3, 4, 1, None, None, FAKE, 1, 512, FAKE, ws, None), -2, "gdn heads")

    # decode layout
    for rows, cols in ((1, 16), (34816, 5120), (5, 8192), (5, 8208), (0, 16)):
        L.nvfp4_decode_weight_bytes(rows, cols)
    L.nvfp4_decode_weight_pack.argtypes = [ctypes.POINTER(Tensor), P, ctypes.c_size_t, P]
    nb = L.nvfp4_decode_weight_bytes(96, 256)
    expect(L.nvfp4_decode_weight_pack(ctypes.byref(w), FAKE, nb, None), 0, "pack")
    expect(L.nvfp4_decode_weight_pack(ctypes.byref(w), FAKE, nb - 1, None), -8, "pack short")
    dw = DecodeWeight(FAKE, 96, 256)
    gdc = L.nvfp4_gemm_decode
    gdc.argtypes = [ctypes.POINTER(Tensor), ctypes.POINTER(DecodeWeight), I32, P, P, ctypes.POINTER(Gate), P, I32,
                    I64, P]
    expect(gdc(ctypes.byref(a), ctypes.byref(dw), 3, offsets(0, 32, 64, 96), FAKE,
               ctypes.byref(Gate(1, 2, FAKE, FAKE)), FAKE, 0, 96, None), 0, "gemm_decode")
    ld = L.nvfp4_linear_decode
    ld.argtypes = [P, I32, I64, I64, P, ctypes.POINTER(DecodeWeight), I32, P, P, ctypes.POINTER(Gate), P, I32, I64,
                   P]
    expect(ld(FAKE, 0, 8, 256, FAKE, ctypes.byref(dw), 1, offsets(0, 96), FAKE, None, FAKE, 0, 96, None), 0,
           "linear_decode")
    expect(ld(FAKE, 0, 17, 256, FAKE, ctypes.byref(dw), 1, offsets(0, 96), FAKE, None, FAKE, 0, 96, None), -2,
           "linear_decode rows")

    for code in range(-12, 2):
        L.nvfp4_status_string(code)
    L.nvfp4_version()
    if L.nvfp4_stub_calls() < 30:
        raise SystemExit(f"only {L.nvfp4_stub_calls()} launcher calls reached the stubs")
    print(f"sanitized ABI driver ok: {checks} checks, {L.nvfp4_stub_calls()} launcher calls")


if __name__ == "__main__":
    main(sys.argv[1])
