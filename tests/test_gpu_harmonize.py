"""GPU parity for the checkpoint-side scale harmonization: block scales
bit-exact against the oracle (in and out of place, ragged K, many
segments), and the harmonized 32K GDN in-projection served with one global
scale against the oracle's GEMM on the harmonized weight, with the mismatch
it repairs measured beside it."""
import numpy as np
import pytest
import torch

import bit_linear_layer_amd as nv
import workloads as W
from oracle import nvfp4_oracle as O
from tests.gpu_util import DEV, assert_close, host_q, say, weight_segments

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows,cols,nseg", [(1, 16, 1), (37, 208, 3), (1000, 5120, 16)])
@pytest.mark.parametrize("in_place", [False, True])
def test_harmonize_scales_exact(rows, cols, nseg, in_place):
    say(f"harmonize {rows}x{cols} segs={nseg} in_place={in_place}")
    rng = np.random.default_rng(rows + nseg)
    cuts = np.sort(rng.choice(np.arange(1, rows), size=nseg - 1, replace=False)) if nseg > 1 else []
    offs = [0, *[int(c) for c in cuts], rows]
    w = nv.empty_nvfp4(rows, cols, DEV)
    sc = rng.integers(0, 0x7F, size=(rows, cols // 16)).astype(np.uint8)
    w.scales[:, : cols // 16].copy_(torch.from_numpy(sc))
    seg_g = (10.0 ** rng.uniform(-5, -1, nseg)).astype(np.float32)
    if nseg > 2:
        seg_g[1] = seg_g[0] / 8  # a power-of-two ratio
    sg = torch.from_numpy(seg_g).to(DEV)
    out = w.scales if in_place else torch.empty_like(w.scales)
    g = torch.empty(1, dtype=torch.float32, device=DEV)
    nv.nvfp4_harmonize_scales(w, offs, sg, out, g)
    torch.cuda.synchronize()
    ref, G = O.harmonize_scales(sc, offs, seg_g)
    assert g.cpu().numpy()[0] == G
    assert np.array_equal(out[:, : cols // 16].cpu().numpy(), ref)


def test_harmonized_gdn_in_proj_served_with_one_scale():
    """32768 x 16480 x 5120, six modules with their own scales, gates on b/a.
    Harmonized and served with one global scale: parity against the oracle
    GEMM on the harmonized weight (sampled rows).  Against the per-module
    (per-segment epilogue) result: every module within the scale rounding
    (<= 2^-4 relative), while serving module q's scale for every column (the
    mismatch) is off by exactly |g_q/g_s - 1|."""
    say("harmonize gdn in-proj 32768")
    wl = W.gdn_in_proj()
    x = wl.x.to(DEV)
    wq, offs, sg = weight_segments([(n, t.to(DEV)) for n, t in wl.weights])
    a = nv.quantize(x)
    hw = nv.harmonize_scales(wq, offs, sg)
    n = len(offs) - 1
    per_module = nv.gemm_fused_segments(a, wq, offs, sg, out_dtype=torch.float32)
    harmonized = nv.gemm(a, hw, out_dtype=torch.float32)
    mismatch = nv.gemm_fused_segments(a, wq, offs, sg[:1].repeat(n), out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 32767], np.random.default_rng(9).integers(0, 32768, 62)]))
    rt = torch.from_numpy(rows).to(DEV)
    ac, as_, ag = host_q(a)
    hc = hw.codes[:, :2560].cpu().numpy()
    hs = hw.scales[:, :320].cpu().numpy()
    ref, tol = O.gemm(ac[rows], as_[rows], ag, hc, hs, hw.global_scale.cpu().numpy()[0], 5120)
    assert_close(harmonized[rt], ref, tol, "f32", "harmonized gemm")
    pm = per_module[rt].cpu().numpy().astype(np.float64)
    hm = harmonized[rt].cpu().numpy().astype(np.float64)
    mm = mismatch[rt].cpu().numpy().astype(np.float64)
    g = sg.cpu().numpy()
    for s in range(n):
        c = slice(offs[s], offs[s + 1])
        e_h = np.linalg.norm(hm[:, c] - pm[:, c]) / np.linalg.norm(pm[:, c])
        e_m = np.linalg.norm(mm[:, c] - pm[:, c]) / np.linalg.norm(pm[:, c])
        assert e_h <= 2.0 ** -4
        assert e_m == pytest.approx(abs(float(g[0]) / float(g[s]) - 1.0), rel=1e-4, abs=1e-6)
