"""GPU parity for the MLP glue (SiLU*mul, amax partials feeding the next
quantization) and the MLP pair chain, checked stage by stage: each stage's
oracle runs on the GPU's own output of the previous stage."""
import numpy as np
import pytest
import torch

import bit_linear_layer_amd as nv
import workloads as W
from oracle import nvfp4_oracle as O
from tests.gpu_util import (DEV, assert_close, assert_quant_exact, host_q, oracle_weight,
                            quantize_dev, say, weight_segments)

pytestmark = pytest.mark.gpu


def bf16_ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """|a - b| in bf16 ulps, via order-preserving integer images."""
    def ordered(v):
        bits = (np.asarray(v, dtype=np.float32).view(np.uint32) >> 16).astype(np.int64)
        return np.where(bits & 0x8000, -(bits & 0x7FFF), bits)
    return np.abs(ordered(a) - ordered(b))


@pytest.mark.parametrize("rows,inter", [(1, 16), (7, 48), (64, 1024), (300, 17408 // 16)])
def test_silu_mul_within_one_bf16_ulp(rows, inter):
    say(f"silu_mul {rows}x{inter}")
    rng = np.random.default_rng(rows + inter)
    gu = W.to_bf16(rng.standard_normal((rows, 2 * inter)) * 6).to(DEV)
    ws = nv.workspace_for(rows, inter)
    h = nv.silu_mul(gu, amax_workspace=ws)
    torch.cuda.synchronize()
    g = W.bf16_to_f32_numpy(gu)
    ref = O.silu_mul(g[:, :inter].astype(np.float64), g[:, inter:].astype(np.float64))
    got = W.bf16_to_f32_numpy(h)
    d = bf16_ulp_distance(got, ref)
    assert d.max() <= 1, f"max distance {d.max()} ulp"
    # the amax partials feed a quantization that needs no amax pass
    q = nv.quantize(h, workspace=ws, amax_precomputed=True)
    assert_quant_exact(h, q)


def test_silu_mul_extreme_inputs():
    say("silu_mul extremes")
    vals = np.array([-200, -100, -90, -88, -20, -1e-3, 0, 1e-3, 20, 88, 100, 200], dtype=np.float64)
    g = np.tile(vals, (2, 4))[:, :48]
    u = np.full_like(g, 1.5)
    gu = W.to_bf16(np.concatenate([g, u], axis=1)).to(DEV)
    h = nv.silu_mul(gu)
    torch.cuda.synchronize()
    gf = W.bf16_to_f32_numpy(gu)
    ref = O.silu_mul(gf[:, :48].astype(np.float64), gf[:, 48:].astype(np.float64))
    assert bf16_ulp_distance(W.bf16_to_f32_numpy(h), ref).max() <= 1


def test_mlp_pair_chain_sampled_rows():
    """8192-token MLP pair (gate_up [34816, 5120] two segments, SiLU*mul,
    re-quantization, down [5120, 17408]), each stage against the oracle on
    the GPU's previous-stage output, on 512 sampled rows (the first and
    last 256-row tiles' edges included)."""
    say("mlp pair 8192 chain")
    wl = W.mlp_pair()
    x = wl.x.to(DEV)
    wgu, offs, sg = weight_segments([(n, w.to(DEV)) for n, w in wl.weights])
    wd, doffs, dg = weight_segments([("down", wl.extra["w_down"].to(DEV))])
    inter = offs[1]
    a = quantize_dev(x)
    gu = nv.gemm_fused_segments(a, wgu, offs, sg, out_dtype=torch.bfloat16)
    ws = nv.workspace_for(x.shape[0], inter)
    h = nv.silu_mul(gu, amax_workspace=ws)
    hq = nv.quantize(h, workspace=ws, amax_precomputed=True)
    out = nv.gemm_fused_segments(hq, wd, doffs, dg, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 7935, 7936, 8191],
                                     np.random.default_rng(3).choice(8192, 505, replace=False)]))
    rt = torch.from_numpy(rows).to(DEV)
    # stage 1: X quantization (sampled rows, g of the whole tensor)
    assert_quant_exact(x, a, rows=rows)
    # stage 2: gate_up GEMM
    ac, as_, ag = host_q(a)
    wc, wsc, g_gu = oracle_weight(wgu, offs, sg)
    ref, tol = O.fused_segments(ac[rows], as_[rows], ag, wc, wsc, offs, g_gu, 5120)
    assert_close(gu[rt], ref, tol, "bf16", "gate_up")
    # stage 3: SiLU*mul on the GPU's gate_up
    g = W.bf16_to_f32_numpy(gu[rt])
    href = O.silu_mul(g[:, :inter].astype(np.float64), g[:, inter:].astype(np.float64))
    assert bf16_ulp_distance(W.bf16_to_f32_numpy(h[rt]), href).max() <= 1
    # stage 4: h quantization
    assert_quant_exact(h, hq, rows=rows)
    # stage 5: down GEMM on the GPU's quantized h
    hc, hs, hg = host_q(hq)
    dc, ds, g_d = oracle_weight(wd, doffs, dg)
    ref, tol = O.fused_segments(hc[rows], hs[rows], hg, dc, ds, doffs, g_d, inter)
    assert_close(out[rt], ref, tol, "bf16", "down")
