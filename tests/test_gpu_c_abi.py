"""A linear layer driven from plain C through the C ABI alone (no Python
binding and no torch in that process): tests/cabi/linear_layer.c, built by
__graft_entry__.build(), quantizes the weight and the activations with
dynamic global scales and multiplies; its outputs against the oracle
(activation codes, scales and global scale bit for bit, the GEMM within
1e-5 * sum|a*w|)."""
import os
import subprocess

import numpy as np
import pytest
import torch

import workloads as W
from oracle import nvfp4_oracle as O
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "cabi", "linear_layer")


@pytest.mark.parametrize("m,n,k", [(96, 272, 640), (8, 1040, 1280)])
def test_linear_layer_from_plain_c(tmp_path, m, n, k):
    if not os.path.exists(EXE):
        pytest.fail("tests/cabi/linear_layer is not built (run __graft_entry__.build())")
    say(f"C ABI linear layer {m}x{n}x{k}")
    rng = np.random.default_rng(m + n + k)
    x = W.to_bf16(rng.standard_normal((m, k)) * 3.0)
    w = W.to_bf16(rng.standard_normal((n, k)) * 0.02)
    (tmp_path / "x.bin").write_bytes(x.view(torch.int16).numpy().tobytes())
    (tmp_path / "w.bin").write_bytes(w.view(torch.int16).numpy().tobytes())
    r = subprocess.run([EXE, str(tmp_path), str(m), str(n), str(k)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    codes = np.fromfile(tmp_path / "a_codes.bin", dtype=np.uint8).reshape(m, k // 2)
    scales = np.fromfile(tmp_path / "a_scales.bin", dtype=np.uint8).reshape(m, k // 16)
    g = np.fromfile(tmp_path / "a_g.bin", dtype=np.float32)[0]
    out = np.fromfile(tmp_path / "out.bin", dtype=np.float32).reshape(m, n)

    xs, ws = W.bf16_to_f32_numpy(x), W.bf16_to_f32_numpy(w)
    oc, osc, og = O.quantize(xs)
    assert g.view(np.uint32) == np.float32(og).view(np.uint32)
    assert np.array_equal(codes, oc) and np.array_equal(scales, osc)
    wc, wsc, wg = O.quantize(ws)
    ref, tol = O.gemm(oc, osc, og, wc, wsc, wg, k)
    err = np.abs(out.astype(np.float64) - ref)
    assert np.all(err <= tol), f"max err/tol {np.max(err / np.maximum(tol, 1e-300)):.3f}"
