"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare with the oracle on the same inputs."""
from __future__ import annotations

import sys

import numpy as np
import torch

import bit_linear_layer_amd as nv
from oracle import nvfp4_oracle as O
from workloads import bf16_to_f32_numpy

DEV = "cuda"


def say(msg: str) -> None:
    """Name the case before a GPU step (survives a box that dies mid-run)."""
    print(msg, file=sys.stderr, flush=True)


def host_q(q: nv.NVFP4Tensor):
    """NVFP4Tensor -> (codes [R, K/2], scales [R, K/16], g) numpy, padding stripped."""
    torch.cuda.synchronize()
    codes = q.codes[:, : q.cols // 2].cpu().numpy()
    scales = q.scales[:, : q.cols // 16].cpu().numpy()
    g = np.float32(q.global_scale.cpu().numpy()[0])
    return codes, scales, g


def x_f32(x: torch.Tensor) -> np.ndarray:
    if x.dtype == torch.bfloat16:
        return bf16_to_f32_numpy(x)
    return x.detach().cpu().numpy().astype(np.float32)


def assert_quant_exact(x: torch.Tensor, q: nv.NVFP4Tensor, g=None, rows=None):
    """Bit-exact comparison of the GPU quantization with the oracle's.
    rows: optional row indices to compare (g must then be given or the
    whole tensor's amax used through the oracle on all rows)."""
    codes, scales, gg = host_q(q)
    xs = x_f32(x)
    if g is None:
        g_ref = O.global_scale(np.abs(xs).max()) if xs.size else np.float32(0)
    else:
        g_ref = np.float32(g)
    assert gg.view(np.uint32) == np.float32(g_ref).view(np.uint32), (gg, g_ref)
    sel = slice(None) if rows is None else rows
    oc, os_, og = O.quantize(xs[sel], g_ref)
    bad = np.argwhere(oc != codes[sel])
    assert bad.size == 0, f"{len(bad)} code bytes differ, first at {bad[:5].tolist()}"
    bad = np.argwhere(os_ != scales[sel])
    assert bad.size == 0, f"{len(bad)} scale bytes differ, first at {bad[:5].tolist()}"


def assert_close(out: torch.Tensor, ref: np.ndarray, tol: np.ndarray, out_dtype: str, what="gemm"):
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    allowed = O.output_tolerance(ref, tol, out_dtype)
    err = np.abs(o - ref)
    bad = np.argwhere(~(err <= allowed))
    if bad.size:
        i, j = bad[0]
        raise AssertionError(f"{what}: {len(bad)} of {err.size} elements outside tolerance; first "
                             f"[{i},{j}] got {o[i, j]!r} ref {ref[i, j]!r} allowed {allowed[i, j]!r}")
    return float(np.max(err / np.maximum(allowed, 1e-300)))


def quantize_dev(x: torch.Tensor, static: float | None = None) -> nv.NVFP4Tensor:
    if static is None:
        return nv.quantize(x)
    return nv.quantize(x, static_scale=torch.tensor([static], dtype=torch.float32, device=x.device))


def weight_segments(segs, device=DEV):
    """Quantize each bf16 weight segment with its own dynamic global scale
    into one concatenated NVFP4 tensor.  Returns (w, offsets, seg_g)."""
    rows = sum(w.shape[0] for _, w in segs)
    k = segs[0][1].shape[1]
    wq = nv.empty_nvfp4(rows, k, device)
    seg_g = torch.empty(len(segs), dtype=torch.float32, device=device)
    ws = nv.workspace_for(max(w.shape[0] for _, w in segs), k, device)
    offs = [0]
    for s, (_, w) in enumerate(segs):
        r0 = offs[-1]
        part = wq.row_slice(r0, r0 + w.shape[0])
        part = nv.NVFP4Tensor(part.codes, part.scales, seg_g[s:s + 1], part.rows, part.cols)
        nv.nvfp4_quantize(w.to(device), part, nv.SCALE_DYNAMIC, ws)
        offs.append(r0 + w.shape[0])
    return wq, offs, seg_g


def oracle_weight(wq: nv.NVFP4Tensor, offs, seg_g):
    torch.cuda.synchronize()
    codes = wq.codes[:, : wq.cols // 2].cpu().numpy()
    scales = wq.scales[:, : wq.cols // 16].cpu().numpy()
    return codes, scales, seg_g.cpu().numpy()
