"""The C-ABI layer (api.hip) built as host C++ under AddressSanitizer and
UBSan, with stub launchers in place of the kernels, driven through every
entry point's valid and rejection paths on the CPU (no GPU).  Any sanitizer
report fails the test."""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
GXX = shutil.which("g++")


def sanitizer_runtime():
    out = subprocess.run([GXX, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


@pytest.mark.skipif(GXX is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"),
                    reason="needs g++ and the HIP headers")
def test_c_abi_under_asan_and_ubsan(tmp_path):
    asan = sanitizer_runtime()
    if asan is None:
        pytest.skip("no libasan for g++")
    flags = ["-std=c++17", "-O1", "-g", "-fPIC", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__=1", "-I/opt/rocm/include",
             "-I" + os.path.join(ROOT, "include")]
    objs = []
    for src, lang in ((os.path.join(ROOT, "bit_linear_layer_amd", "csrc", "api.hip"), "c++"),
                      (os.path.join(HERE, "sanitize", "stub_launchers.cpp"), "c++")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        subprocess.run([GXX, *flags, "-x", lang, "-c", src, "-o", obj], check=True)
        objs.append(obj)
    lib = str(tmp_path / "libnvfp4_sanitized.so")
    subprocess.run([GXX, "-shared", "-fsanitize=address,undefined", *objs, "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib", "-o", lib], check=True)
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, os.path.join(HERE, "sanitize", "abi_driver.py"), lib], env=env,
                       capture_output=True, text=True, timeout=300)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-4000:]
    assert "sanitized ABI driver ok" in r.stdout
    assert "ERROR: AddressSanitizer" not in report and "runtime error" not in report
