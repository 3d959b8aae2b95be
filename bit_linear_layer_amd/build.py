"""Build the HIP library libnvfp4.so in-tree for gfx950 (hipcc, no JIT).

Each source compiles to its own object in parallel (every kernel is
launched from its own translation unit, so no relocatable device code is
needed), then one link makes the shared library.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
SOURCES = ["api.hip", "quant.hip", "gemm.hip", "gemm_skinny.hip", "gemm_decode.hip", "glue.hip", "kv_fp8.hip", "harmonize.hip",
           "gdn.hip", "noalloc.hip"]
LIB = os.path.join(PKG, "libnvfp4.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # Keep the compiler from forming packed-fp32 VALU ops in device code.
    # The driver forwards -Xclang to the host pass as well, which does not
    # know the feature and says so once per source; that one line is
    # dropped from the output below (tests/test_build.py checks the built
    # code object for packed-fp32 instructions).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]
_HOST_FEATURE_NOTE = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"


def _run(cmd: list[str]) -> None:
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if l.strip() != _HOST_FEATURE_NOTE)
    if out.strip():
        print(out, flush=True)
    if r.returncode != 0:
        raise subprocess.CalledProcessError(r.returncode, cmd)


def build(verbose: bool = True, jobs: int | None = None) -> str:
    os.makedirs(OBJ, exist_ok=True)
    objs = [os.path.join(OBJ, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    cmds = [[HIPCC, *FLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    if verbose:
        print(" ".join(cmds[0][:-4]) + " -c <source> -o <object>   # " + " ".join(SOURCES), flush=True)
    jobs = jobs or min(len(cmds), os.cpu_count() or 1, 16)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(_run, cmds))
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"])
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
