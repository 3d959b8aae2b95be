"""GPU parity for the fused gated-MLP first half (nvfp4_gemm_swiglu):

* bit for bit the unfused chain (gate_up GEMM to bf16, SiLU*mul, quantize
  of h with precomputed amax partials), at ragged small shapes in both tile
  configurations and at the full 8192-token MLP size;
* against the oracle end to end, within a bound carried through the bf16
  roundings of gate and up and the SiLU (a property that holds whatever the
  accumulation order);
* the static-scale NVFP4 output bit-exact against the oracle's quantization
  of the same h, including scales that saturate and scales that flush
  blocks to zero."""
import numpy as np
import pytest
import torch

import bit_linear_layer_amd as nv
import workloads as W
from oracle import nvfp4_oracle as O
from tests.gpu_util import (DEV, assert_quant_exact, host_q, oracle_weight, quantize_dev, say,
                            weight_segments)

pytestmark = pytest.mark.gpu


def make_case(m, inter, k, seed):
    rng = np.random.default_rng(seed)
    x = W.to_bf16(W.outlier_activations(rng, m, k, heavy=True, n_outlier=3, factor=20.0)).to(DEV)
    wg = W.to_bf16(W.normal_weight(rng, inter, k, 0.02)).to(DEV)
    wu = W.to_bf16(W.normal_weight(rng, inter, k, 0.03)).to(DEV)
    w, offs, sg = weight_segments([("gate", wg), ("up", wu)])
    return quantize_dev(x), w, offs, sg


def unfused(a, w, offs, sg):
    inter = offs[1]
    gu = nv.gemm_fused_segments(a, w, offs, sg, out_dtype=torch.bfloat16)
    ws = nv.workspace_for(a.rows, inter)
    h = nv.silu_mul(gu, amax_workspace=ws)
    hq = nv.quantize(h, workspace=ws, amax_precomputed=True)
    return gu, h, hq


def fused(a, w, sg):
    inter = w.rows // 2
    ws = nv.workspace_for(a.rows, inter)
    h = nv.gemm_swiglu(a, w, sg, amax_workspace=ws)
    hq = nv.quantize(h, workspace=ws, amax_precomputed=True)
    return h, hq


def assert_same_nvfp4(p, q):
    torch.cuda.synchronize()
    assert torch.equal(p.global_scale, q.global_scale)
    assert torch.equal(p.codes[:, : p.cols // 2], q.codes[:, : q.cols // 2])
    assert torch.equal(p.scales[:, : p.cols // 16], q.scales[:, : q.cols // 16])


def silu64(x):
    return x * O.sigmoid(x)


def swiglu_bound(g_ref, g_tol, u_ref, u_tol):
    """Bound on |h - silu(g_ref) * u_ref| for h = bf16(silu(bf16(g)) * bf16(u))
    with |g - g_ref| <= g_tol, |u - u_ref| <= u_tol.  bf16 rounding moves a
    value by <= 2^-8 of itself; |silu'| <= 1.1 everywhere; the fp32
    evaluation of silu and of the product adds a few fp32 ulps (1e-6)."""
    eps = 2.0 ** -8
    dg = g_tol + eps * (np.abs(g_ref) + g_tol)
    du = u_tol + eps * (np.abs(u_ref) + u_tol)
    s = silu64(g_ref)
    h = s * u_ref
    dh = 1.1 * dg * (np.abs(u_ref) + du) + np.abs(s) * du
    dh += 1e-6 * (np.abs(s) + 1.1 * dg) * (np.abs(u_ref) + du)
    return h, dh + eps * (np.abs(h) + dh)


# (M, inter, K): tiny and ragged shapes run the 128-row tiles; 2000/2048 x
# 3456 fills the chip with 256 x 128 tiles (the large configuration); K
# values 208, 144, 320 leave ragged last K tiles, 256, 384 and 640 are whole
# K tiles (the software-pipelined kernel, 128-row and 256-row tiles).
SHAPES = [(5, 48, 64), (300, 272, 208), (1024, 1024, 320), (2000, 3456, 208), (2048, 3456, 144),
          (2000, 3456, 256), (2048, 3456, 640), (1024, 1024, 256), (300, 272, 384)]


@pytest.mark.parametrize("m,inter,k", SHAPES)
def test_swiglu_equals_unfused_chain(m, inter, k):
    say(f"swiglu vs unfused {m}x{inter}x{k}")
    a, w, offs, sg = make_case(m, inter, k, seed=m + inter + k)
    _, h0, hq0 = unfused(a, w, offs, sg)
    h1, hq1 = fused(a, w, sg)
    torch.cuda.synchronize()
    diff = (h0.view(torch.int16) != h1.view(torch.int16)).sum().item()
    assert diff == 0, f"{diff} h elements differ from the unfused chain"
    assert_same_nvfp4(hq0, hq1)


@pytest.mark.parametrize("m,inter,k", [(300, 272, 208), (2000, 3456, 208), (2000, 3456, 256), (300, 272, 384)])
def test_swiglu_against_oracle(m, inter, k):
    say(f"swiglu vs oracle {m}x{inter}x{k}")
    a, w, offs, sg = make_case(m, inter, k, seed=7 * m + k)
    ws = nv.workspace_for(m, inter)
    h = nv.gemm_swiglu(a, w, sg, amax_workspace=ws)
    hq = nv.quantize(h, workspace=ws, amax_precomputed=True)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, m - 1], np.random.default_rng(1).integers(0, m, 60)]))
    ac, as_, ag = host_q(a)
    wc, wsc, g = oracle_weight(w, offs, sg)
    ref, tol = O.fused_segments(ac[rows], as_[rows], ag, wc, wsc, offs, g, k)
    href, bound = swiglu_bound(ref[:, :inter], tol[:, :inter], ref[:, inter:], tol[:, inter:])
    got = W.bf16_to_f32_numpy(h)[rows].astype(np.float64)
    bad = np.argwhere(~(np.abs(got - href) <= bound))
    assert bad.size == 0, f"{len(bad)} h elements outside the bound, first {bad[:3].tolist()}"
    # the fused amax partials give h's dynamic global scale
    assert_quant_exact(h, hq)


@pytest.mark.parametrize("m,inter,k", [(300, 272, 208), (2048, 3456, 144), (300, 272, 384), (2000, 3456, 256)])
@pytest.mark.parametrize("gscale", [1.0, 0.05, 40.0])
def test_swiglu_static_quantized_output(m, inter, k, gscale):
    """h_q with a calibrated scale: gscale 1 uses h's own dynamic scale,
    0.05 saturates most block scales at 448, 40 flushes small blocks."""
    say(f"swiglu static {m}x{inter}x{k} x{gscale}")
    a, w, offs, sg = make_case(m, inter, k, seed=m + 3 * k)
    ws = nv.workspace_for(m, inter)
    h = nv.gemm_swiglu(a, w, sg, amax_workspace=ws)
    hq_dyn = nv.quantize(h, workspace=ws, amax_precomputed=True)
    torch.cuda.synchronize()
    g = hq_dyn.global_scale * gscale
    both = nv.empty_nvfp4(m, inter, DEV)
    both.global_scale.copy_(g)
    h2 = torch.empty_like(h)
    nv.nvfp4_gemm_swiglu(a, w, sg, h=h2, h_q=both)
    only = nv.gemm_swiglu_quantized(a, w, sg, g)
    torch.cuda.synchronize()
    assert torch.equal(h.view(torch.int16), h2.view(torch.int16))
    assert_same_nvfp4(both, only)
    assert_quant_exact(h, only, g=float(g.cpu().numpy()[0]))


def test_swiglu_mlp_size_equals_unfused_and_oracle_rows():
    """The 8192-token MLP pair's gate_up (34816 x 5120, two segments)."""
    say("swiglu mlp 8192 full size")
    wl = W.mlp_pair()
    x = wl.x.to(DEV)
    w, offs, sg = weight_segments([(n, t.to(DEV)) for n, t in wl.weights])
    a = quantize_dev(x)
    gu, h0, hq0 = unfused(a, w, offs, sg)
    del gu
    h1, hq1 = fused(a, w, sg)
    torch.cuda.synchronize()
    assert torch.equal(h0.view(torch.int16), h1.view(torch.int16))
    assert_same_nvfp4(hq0, hq1)
    inter = offs[1]
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 7935, 7936, 8191],
                                     np.random.default_rng(5).integers(0, 8192, 121)]))
    ac, as_, ag = host_q(a)
    wc, wsc, g = oracle_weight(w, offs, sg)
    ref, tol = O.fused_segments(ac[rows], as_[rows], ag, wc, wsc, offs, g, 5120)
    href, bound = swiglu_bound(ref[:, :inter], tol[:, :inter], ref[:, inter:], tol[:, inter:])
    got = W.bf16_to_f32_numpy(h1[torch.from_numpy(rows).to(DEV)]).astype(np.float64)
    assert np.all(np.abs(got - href) <= bound)
