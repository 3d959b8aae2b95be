"""The built library's gfx950 code objects hold no packed-fp32 VALU
instructions (the build turns the feature off for device code), and every
kernel source is in the build."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "bit_linear_layer_amd", "libnvfp4.so")
OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"


def test_every_source_is_built():
    from bit_linear_layer_amd import build
    csrc = os.path.join(ROOT, "bit_linear_layer_amd", "csrc")
    hip = sorted(f for f in os.listdir(csrc) if f.endswith(".hip"))
    assert sorted(build.SOURCES) == hip


@pytest.mark.skipif(not os.path.exists(LIB) or not os.path.exists(OBJDUMP), reason="library or llvm-objdump missing")
def test_no_packed_fp32_instructions(tmp_path):
    lib = tmp_path / "lib.so"
    shutil.copy(LIB, lib)
    subprocess.run([OBJDUMP, "--offloading", str(lib)], check=True, cwd=tmp_path, capture_output=True)
    objs = [p for p in tmp_path.iterdir() if p.name.endswith("gfx950")]
    assert objs, "no gfx950 code object in the library"
    packed = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")
    mfma = 0
    for p in objs:
        dis = subprocess.run([OBJDUMP, "-d", str(p)], check=True, capture_output=True, text=True).stdout
        mfma += dis.count("v_mfma")
        hits = [l for l in dis.splitlines() if packed.search(l)]
        assert not hits, f"{p.name}: {hits[:3]}"
    assert mfma > 0, "the disassembly holds no MFMA at all"
