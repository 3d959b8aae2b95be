"""The built library's gfx950 code objects hold no packed-fp32 VALU
instructions (the build turns the feature off for device code), the
streaming outputs are written with nontemporal stores, and every kernel
source is in the build."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "bit_linear_layer_amd", "libnvfp4.so")
OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"

needs_lib = pytest.mark.skipif(not os.path.exists(LIB) or not os.path.exists(OBJDUMP),
                               reason="library or llvm-objdump missing")


def test_every_source_is_built():
    from bit_linear_layer_amd import build
    csrc = os.path.join(ROOT, "bit_linear_layer_amd", "csrc")
    hip = sorted(f for f in os.listdir(csrc) if f.endswith(".hip"))
    assert sorted(build.SOURCES) == hip


@pytest.fixture(scope="module")
def disassembly(tmp_path_factory):
    """{code object name: disassembly text} of the library's gfx950 code objects."""
    tmp = tmp_path_factory.mktemp("objs")
    lib = tmp / "lib.so"
    shutil.copy(LIB, lib)
    subprocess.run([OBJDUMP, "--offloading", str(lib)], check=True, cwd=tmp, capture_output=True)
    objs = [p for p in tmp.iterdir() if p.name.endswith("gfx950")]
    assert objs, "no gfx950 code object in the library"
    return {p.name: subprocess.run([OBJDUMP, "-d", str(p)], check=True, capture_output=True, text=True).stdout
            for p in objs}


def functions(disassembly):
    """{symbol: [instruction lines]} over all code objects."""
    out, cur = {}, None
    for text in disassembly.values():
        for line in text.splitlines():
            m = re.match(r"^[0-9a-f]+ <(.+)>:$", line)
            if m:
                cur = out.setdefault(m.group(1), [])
            elif cur is not None and line.strip():
                cur.append(line)
    return out


@needs_lib
def test_no_packed_fp32_instructions(disassembly):
    packed = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")
    mfma = 0
    for name, dis in disassembly.items():
        mfma += dis.count("v_mfma")
        hits = [l for l in dis.splitlines() if packed.search(l)]
        assert not hits, f"{name}: {hits[:3]}"
    assert mfma > 0, "the disassembly holds no MFMA at all"


@needs_lib
def test_streaming_outputs_use_nontemporal_stores(disassembly):
    fns = functions(disassembly)

    def stores(part):
        found = {n: [l for l in body if "global_store" in l] for n, body in fns.items() if part in n}
        assert found, f"no kernel named like {part}"
        return found

    # the FP8 KV cache and its read-back: every store streams
    for part in ("kv_quant_kernel", "kv_quant_linear_kernel", "kv_dequant_kernel"):
        for name, st in stores(part).items():
            assert st and all(re.search(r"\bnt\b", l) for l in st), f"{name}: {st[:4]}"
    # the quantizer's codes (8 bytes) and scales (1 byte) per block
    for name, st in stores("quantize_kernel").items():
        blk = [l for l in st if "global_store_dwordx2" in l or "global_store_byte" in l]
        assert blk and all(re.search(r"\bnt\b", l) for l in blk), f"{name}: {blk[:4]}"
    # SiLU*mul's h rows
    for name, st in stores("silu_mul_kernel").items():
        assert any("global_store_dwordx4" in l and re.search(r"\bnt\b", l) for l in st), name
    # the pipelined GEMM's staged bf16 tiles
    pipe = stores("gemm_kernel_pipe")
    assert any(any("global_store_dwordx4" in l and re.search(r"\bnt\b", l) for l in st) for st in pipe.values())
