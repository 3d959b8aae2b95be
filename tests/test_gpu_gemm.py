"""GPU parity: W4A4 GEMM, fused segments and the GDN gate epilogue through
the C ABI, against the oracle's float64 GEMM on the same quantized operands
(|err| <= 1e-5 * sum|a*w| per element, plus half a bf16 ulp for bf16)."""
import numpy as np
import pytest
import torch

import bit_linear_layer_amd as nv
import workloads as W
from oracle import nvfp4_oracle as O
from tests.gpu_util import (DEV, assert_close, host_q, oracle_weight, quantize_dev, say,
                            weight_segments)

pytestmark = pytest.mark.gpu


def rand_bf16(seed, rows, cols, scale=1.0, outliers=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)) * scale
    if outliers:
        x[:, rng.choice(cols, outliers, replace=False)] *= 60
    return W.to_bf16(x).to(DEV)


def run_gemm(x, w, out_dtype):
    a = quantize_dev(x)
    wq = quantize_dev(w)
    out = nv.gemm(a, wq, out_dtype=out_dtype)
    ac, as_, ag = host_q(a)
    wc, ws, wg = host_q(wq)
    ref, tol = O.gemm(ac, as_, ag, wc, ws, wg, x.shape[1])
    return out, ref, tol


SHAPES = [(1, 48, 16), (8, 130, 32), (17, 64, 48), (33, 257, 144), (100, 300, 256),
          (300, 520, 1040), (256, 256, 128), (513, 384, 640), (32, 128, 256), (64, 96, 5120)]


@pytest.mark.parametrize("m,n,k", SHAPES, ids=lambda v: str(v))
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_gemm_shapes(m, n, k, out_dtype):
    say(f"gemm {m}x{n}x{k} {out_dtype}")
    x = rand_bf16(m * 31 + n, m, k, outliers=min(2, k // 16))
    w = rand_bf16(n * 17 + k, n, k, 0.02)
    out, ref, tol = run_gemm(x, w, torch.float32 if out_dtype == "f32" else torch.bfloat16)
    assert_close(out, ref, tol, out_dtype)


def test_tiny_config_fp32():
    say("gemm tiny 32x128x256")
    wl = W.tiny()
    out, ref, tol = run_gemm(wl.x.to(DEV), wl.weights[0][1].to(DEV), torch.float32)
    assert_close(out, ref, tol, "f32")


def test_act_quant_gemm_full_size():
    say("gemm act_quant_gemm 4096x5120x5120")
    wl = W.act_quant_gemm()
    out, ref, tol = run_gemm(wl.x.to(DEV), wl.weights[0][1].to(DEV), torch.bfloat16)
    assert_close(out, ref, tol, "bf16")


def test_accumulation_stress_all_positive():
    """All-positive operands at K = 17408: no cancellation, the fp32
    accumulation error is at its relative worst."""
    say("gemm all-positive K=17408")
    rng = np.random.default_rng(5)
    x = W.to_bf16(np.abs(rng.standard_normal((64, 17408)))).to(DEV)
    w = W.to_bf16(np.abs(rng.normal(0, 0.02, (256, 17408)))).to(DEV)
    out, ref, tol = run_gemm(x, w, torch.float32)
    ratio = assert_close(out, ref, tol, "f32")
    say(f"  worst err / tolerance = {ratio:.3f}")


def test_output_canaries_and_determinism():
    """Stores stay inside [M, N] of a strided output, and two runs agree
    bit for bit."""
    say("gemm canaries")
    m, n, k = 77, 200, 384
    x = rand_bf16(1, m, k)
    w = rand_bf16(2, n, k, 0.02)
    a, wq = quantize_dev(x), quantize_dev(w)
    big = torch.full((m + 5, n + 24), 12345.0, dtype=torch.float32, device=DEV)
    view = big[:m, :n]
    nv.nvfp4_gemm(a, wq, view)
    torch.cuda.synchronize()
    assert torch.all(big[m:] == 12345.0) and torch.all(big[:, n:] == 12345.0)
    again = nv.gemm(a, wq, out_dtype=torch.float32)
    assert torch.equal(again, view)
    ac, as_, ag = host_q(a)
    wc, ws, wg = host_q(wq)
    ref, tol = O.gemm(ac, as_, ag, wc, ws, wg, k)
    assert_close(view, ref, tol, "f32")


# ------------------------------------------------------------ segments


def small_gdn(m=200, scale_rows=1 / 64, k=512):
    wl = W.gdn_in_proj(seed=0, m=m, k=k, scale_rows=scale_rows)
    x = wl.x.to(DEV)
    wq, offs, seg_g = weight_segments([(n, w.to(DEV)) for n, w in wl.weights])
    return wl, x, wq, offs, seg_g


@pytest.mark.parametrize("k", [512, 272])  # whole K tiles (pipelined kernel) and a ragged last K tile
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_fused_segments_with_gates(out_dtype, k):
    say(f"fused GDN small {out_dtype} k={k}")
    wl, x, wq, offs, seg_g = small_gdn(k=k)
    a = quantize_dev(x)
    gate = dict(b_segment=4, a_segment=5, A_log=wl.extra["A_log"].to(DEV), dt_bias=wl.extra["dt_bias"].to(DEV))
    tdt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    out = nv.gemm_fused_segments(a, wq, offs, seg_g, gate=gate, out_dtype=tdt)
    ac, as_, ag = host_q(a)
    wc, ws, sg = oracle_weight(wq, offs, seg_g)
    ref, tol = O.fused_segments(ac, as_, ag, wc, ws, offs, sg, x.shape[1])
    o = out.float().cpu().numpy()
    # linear segments
    lin = slice(0, offs[4])
    assert_close(out[:, lin], ref[:, lin], tol[:, lin], out_dtype, "fused linear segments")
    # gates
    a_log = wl.extra["A_log"].numpy().astype(np.float64)
    dt_bias = wl.extra["dt_bias"].numpy().astype(np.float64)
    bsl, asl = slice(offs[4], offs[5]), slice(offs[5], offs[6])
    beta, tb, _, _ = O.gate_tolerances(ref[:, bsl], tol[:, bsl], a_log, dt_bias)
    _, _, dec, td = O.gate_tolerances(ref[:, asl], tol[:, asl], a_log, dt_bias)
    assert_close(out[:, bsl], beta, tb, out_dtype, "sigmoid gate")
    assert_close(out[:, asl], dec, td, out_dtype, "decay gate")
    assert np.all(o[:, asl] < 0) and np.all((o[:, bsl] >= 0) & (o[:, bsl] <= 1))


@pytest.mark.parametrize("m", [200, 24, 8])  # 128-row tiles, 32-row tiles, the M <= 16 kernel
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_gates_wide_argument_range(out_dtype, m):
    """The gate epilogue far out in both tails: the b and a segments' global
    scales are raised by powers of two (exact) until their pre-activations
    reach about 256 in magnitude, so sigmoid saturates at 1 and underflows,
    the decay's argument passes the float32 underflow of exp, and both gates
    produce subnormal float32 results."""
    say(f"gates over a wide argument range m={m} {out_dtype}")
    wl, x, wq, offs, seg_g = small_gdn(m=m)
    a = quantize_dev(x)
    ac, as_, ag = host_q(a)
    wc, ws, sg = oracle_weight(wq, offs, seg_g)
    ref0, _ = O.fused_segments(ac, as_, ag, wc, ws, offs, sg, x.shape[1])
    bsl, asl = slice(offs[4], offs[5]), slice(offs[5], offs[6])
    boost = [int(np.floor(np.log2(256.0 / np.abs(ref0[:, sl]).max()))) for sl in (bsl, asl)]
    assert min(boost) >= 0
    seg_g2 = seg_g.clone()
    seg_g2[4] *= 2.0 ** boost[0]
    seg_g2[5] *= 2.0 ** boost[1]
    gate = dict(b_segment=4, a_segment=5, A_log=wl.extra["A_log"].to(DEV), dt_bias=wl.extra["dt_bias"].to(DEV))
    tdt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    out = nv.gemm_fused_segments(a, wq, offs, seg_g2, gate=gate, out_dtype=tdt)
    wc, ws, sg2 = oracle_weight(wq, offs, seg_g2)
    ref, tol = O.fused_segments(ac, as_, ag, wc, ws, offs, sg2, x.shape[1])
    a_log = wl.extra["A_log"].numpy().astype(np.float64)
    dt_bias = wl.extra["dt_bias"].numpy().astype(np.float64)
    # the tails are really reached: sigmoid past underflow, decay arguments
    # past the float32 underflow of exp (-103.9)
    assert ref[:, bsl].min() < -110 and ref[:, bsl].max() > 100
    assert (ref[:, asl] + dt_bias).min() < -110 and (ref[:, asl] + dt_bias).max() > 100
    beta, tb, _, _ = O.gate_tolerances(ref[:, bsl], tol[:, bsl], a_log, dt_bias)
    _, _, dec, td = O.gate_tolerances(ref[:, asl], tol[:, asl], a_log, dt_bias)
    # float32 cannot resolve below 2^-149: a gate value in the subnormal range
    # (or past underflow) carries a few such quanta from its last roundings
    floor = 2.0 ** -147
    assert_close(out[:, bsl], beta, tb + floor, out_dtype, "sigmoid gate, wide range")
    assert_close(out[:, asl], dec, td + floor, out_dtype, "decay gate, wide range")
    o = out.float().cpu().numpy()
    assert np.all(o[:, asl] <= 0) and np.all((o[:, bsl] >= 0) & (o[:, bsl] <= 1))
    assert np.all(np.isfinite(o[:, offs[4]:offs[6]]))


def test_fused_equals_per_segment_gemms():
    say("fused == concat")
    wl, x, wq, offs, seg_g = small_gdn(m=96)
    a = quantize_dev(x)
    fused = nv.gemm_fused_segments(a, wq, offs, seg_g, out_dtype=torch.float32)
    for s in range(len(offs) - 1):
        part = wq.row_slice(offs[s], offs[s + 1])
        part = nv.NVFP4Tensor(part.codes, part.scales, seg_g[s:s + 1], part.rows, part.cols)
        single = nv.gemm(a, part, out_dtype=torch.float32)
        d = (single - fused[:, offs[s]:offs[s + 1]]).abs().max().item()
        scale = single.abs().max().item()
        assert d <= 1e-5 * max(scale, 1e-30), (s, d, scale)


def test_single_global_scale_mismatch_is_detected():
    """Serving the fused weight with one module's global scale (the
    mismatch) puts every other segment off by g_w[0]/g_w[s]."""
    say("fused mismatch negative test")
    wl, x, wq, offs, seg_g = small_gdn(m=64)
    a = quantize_dev(x)
    good = nv.gemm_fused_segments(a, wq, offs, seg_g, out_dtype=torch.float32)
    bad = nv.gemm_fused_segments(a, wq, offs, seg_g[:1].repeat(len(offs) - 1).contiguous(), out_dtype=torch.float32)
    g = seg_g.cpu().numpy()
    off_by_far = 0
    for s in range(1, len(offs) - 1):
        sl = slice(offs[s], offs[s + 1])
        ratio = float(g[0]) / float(g[s])
        assert torch.allclose(bad[:, sl], good[:, sl] * ratio, rtol=1e-5, atol=1e-30)
        if abs(ratio - 1) > 0.05:  # far outside the GEMM tolerance
            off_by_far += 1
            assert not torch.allclose(bad[:, sl], good[:, sl], rtol=1e-3, atol=0)
    assert off_by_far >= 3  # the wide-sigma segments really differ in scale


@pytest.mark.parametrize("k", [272, 256, 384])
def test_column_split_launch_sampled_rows(k):
    """M = 8192, N = 5120 (the MLP down projection's output): 640 tiles of
    256x256 leave a half-empty last wave, so the columns past 4096 run as
    256x128 tiles in a second launch.  K = 272 (ragged last K tile) runs the
    two-wave kernels, K = 256 and 384 the pipelined ones.  192 sampled rows
    against the oracle, every column, both sides of the split."""
    say(f"gemm column split 8192x5120x{k}")
    x = rand_bf16(31, 8192, k)
    w = rand_bf16(32, 5120, k, 0.05)
    a = quantize_dev(x)
    wq = quantize_dev(w)
    out = nv.gemm(a, wq, out_dtype=torch.bfloat16)
    rows = np.unique(np.concatenate([[0, 255, 256, 8191], np.random.default_rng(3).integers(0, 8192, 188)]))
    ac, as_, ag = host_q(a)
    wc, ws, wg = host_q(wq)
    ref, tol = O.gemm(ac[rows], as_[rows], ag, wc, ws, wg, k)
    assert_close(out[torch.from_numpy(rows).to(DEV)], ref, tol, "bf16")


@pytest.mark.parametrize("m,n,k", [(4000, 4000, 256), (4000, 4000, 384), (4096, 4096, 640), (4096, 5120, 256),
                                   (4001, 4000, 384), (8190, 5120, 256)],
                         ids=lambda v: str(v))
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_large_tiles_whole_k_tiles_sampled_rows(m, n, k, out_dtype):
    """Shapes that fill the chip with 256x256 tiles and whose K is a whole
    number of 128-wide K tiles run the software-pipelined one-wave-per-SIMD
    kernel: K = 256 is its shortest case (two K tiles, re-copies from the
    start), 384 and 640 run whole pipelines; ragged M and N tiles.  4096 x
    5120 (the act-quant GEMM's shape) runs one wave of 256x256 tiles on
    columns 0-4095 and 128x128 tiles on the rest; 4001 rows end in a
    partial 32-row fragment; 8190 x 5120 runs 256x256 and 256x128 tiles,
    both with a partial last fragment.  Sampled rows (first and last tile
    rows included) against the oracle, every column."""
    say(f"gemm large pipelined {m}x{n}x{k} {out_dtype}")
    x = rand_bf16(40 + k, m, k, outliers=2)
    w = rand_bf16(41 + k, n, k, 0.02)
    a = quantize_dev(x)
    wq = quantize_dev(w)
    dt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    out = nv.gemm(a, wq, out_dtype=dt)
    rows = np.unique(np.concatenate([[0, 255, 256, 3839, 3840, m - 2, m - 1],
                                     np.random.default_rng(k).integers(0, m, 90)]))
    ac, as_, ag = host_q(a)
    wc, ws, wg = host_q(wq)
    ref, tol = O.gemm(ac[rows], as_[rows], ag, wc, ws, wg, k)
    assert_close(out[torch.from_numpy(rows).to(DEV)], ref, tol, out_dtype)


def padded_nvfp4(rows, cols, extra_codes, extra_scales):
    """An NVFP4 tensor whose code and scale rows are longer than needed."""
    codes = torch.full((rows, cols // 2 + extra_codes), 0x77, dtype=torch.uint8, device=DEV)
    scales = torch.full((rows, cols // 16 + extra_scales), 0x7E, dtype=torch.uint8, device=DEV)
    return nv.NVFP4Tensor(codes, scales, torch.empty(1, dtype=torch.float32, device=DEV), rows, cols)


@pytest.mark.parametrize("m,n,k", [(4096, 4096, 384), (2048, 1024, 256)], ids=lambda v: str(v))
def test_padded_operand_strides_pipelined(m, n, k):
    """Operands whose code and scale rows are padded beyond K (the padding
    holds large nonzero codes and scales that must never be read) on the
    pipelined kernels (256x256 and 128x128 tiles)."""
    say(f"gemm padded strides {m}x{n}x{k}")
    x = rand_bf16(60 + k, m, k, outliers=2)
    w = rand_bf16(61 + k, n, k, 0.02)
    a = padded_nvfp4(m, k, 48, 24)
    wq = padded_nvfp4(n, k, 80, 8)
    ws = nv.workspace_for(max(m, n), k, DEV)
    nv.nvfp4_quantize(x, a, nv.SCALE_DYNAMIC, ws)
    nv.nvfp4_quantize(w, wq, nv.SCALE_DYNAMIC, ws)
    out = nv.gemm(a, wq, out_dtype=torch.float32)
    rows = np.unique(np.concatenate([[0, 255, 256, m - 1], np.random.default_rng(k).integers(0, m, 60)]))
    ac, as_, ag = host_q(a)
    wc, wsc, wg = host_q(wq)
    ref, tol = O.gemm(ac[rows], as_[rows], ag, wc, wsc, wg, k)
    assert_close(out[torch.from_numpy(rows).to(DEV)], ref, tol, "f32")


def test_gdn_in_proj_full_size_sampled_rows():
    """32768 x 16480 x 5120 fused GDN in-projection with the gate epilogue:
    512 sampled rows (the first and last 256-row tiles' edges included),
    every column (all segment boundaries), against the oracle."""
    say("fused GDN 32768x16480x5120 sampled")
    wl = W.gdn_in_proj()
    x = wl.x.to(DEV)
    wq, offs, seg_g = weight_segments([(n, w.to(DEV)) for n, w in wl.weights])
    a = quantize_dev(x)
    gate = dict(b_segment=4, a_segment=5, A_log=wl.extra["A_log"].to(DEV), dt_bias=wl.extra["dt_bias"].to(DEV))
    out = nv.gemm_fused_segments(a, wq, offs, seg_g, gate=gate, out_dtype=torch.bfloat16)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 32511, 32512, 32767],
                                     np.random.default_rng(2).choice(32768, 505, replace=False)]))
    ac, as_, ag = host_q(a)
    wc, ws, sg = oracle_weight(wq, offs, seg_g)
    ref, tol = O.fused_segments(ac[rows], as_[rows], ag, wc, ws, offs, sg, 5120)
    o = out[torch.from_numpy(rows).to(DEV)]
    lin = slice(0, offs[4])
    assert_close(o[:, lin], ref[:, lin], tol[:, lin], "bf16", "GDN q/k/v/z")
    a_log = wl.extra["A_log"].numpy().astype(np.float64)
    dt_bias = wl.extra["dt_bias"].numpy().astype(np.float64)
    bsl, asl = slice(offs[4], offs[5]), slice(offs[5], offs[6])
    beta, tb, _, _ = O.gate_tolerances(ref[:, bsl], tol[:, bsl], a_log, dt_bias)
    _, _, dec, td = O.gate_tolerances(ref[:, asl], tol[:, asl], a_log, dt_bias)
    assert_close(o[:, bsl], beta, tb, "bf16", "b gate")
    assert_close(o[:, asl], dec, td, "bf16", "a gate")


def test_decode_full_size():
    """M = 8 tokens x the fused gate_up weight [34816, 5120] (two segments)."""
    say("decode 8x34816x5120")
    wl = W.decode()
    x = wl.x.to(DEV)
    wq, offs, seg_g = weight_segments([(n, w.to(DEV)) for n, w in wl.weights])
    a = quantize_dev(x)
    out = nv.gemm_fused_segments(a, wq, offs, seg_g, out_dtype=torch.bfloat16)
    ac, as_, ag = host_q(a)
    wc, ws, sg = oracle_weight(wq, offs, seg_g)
    ref, tol = O.fused_segments(ac, as_, ag, wc, ws, offs, sg, 5120)
    assert_close(out, ref, tol, "bf16", "decode")


# ------------------------------------------------- small-M (decode) path

@pytest.mark.parametrize("m,n,k", [(1, 16, 16), (3, 40, 48), (8, 1000, 144), (16, 257, 1040),
                                   (5, 4099, 5120), (8, 700, 5104), (2, 96, 5136), (16, 2048, 4096)],
                         ids=lambda v: str(v))
def test_small_m_shapes(m, n, k):
    """M <= 16 runs the weight-streaming kernel (K <= 5120) or the tiled
    kernel beyond; ragged N, K % 128 != 0 and K % 32 == 16 included."""
    say(f"small-M gemm {m}x{n}x{k}")
    x = rand_bf16(m * 101 + k, m, k, outliers=min(2, k // 16))
    w = rand_bf16(n * 7 + k, n, k, 0.02)
    out, ref, tol = run_gemm(x, w, torch.float32)
    assert_close(out, ref, tol, "f32")


def test_small_m_fused_segments_with_gates():
    say("small-M fused GDN with gates")
    wl, x, wq, offs, seg_g = small_gdn(m=4)
    a = quantize_dev(x)
    gate = dict(b_segment=4, a_segment=5, A_log=wl.extra["A_log"].to(DEV), dt_bias=wl.extra["dt_bias"].to(DEV))
    out = nv.gemm_fused_segments(a, wq, offs, seg_g, gate=gate, out_dtype=torch.float32)
    ac, as_, ag = host_q(a)
    wc, ws, sg = oracle_weight(wq, offs, seg_g)
    ref, tol = O.fused_segments(ac, as_, ag, wc, ws, offs, sg, x.shape[1])
    lin = slice(0, offs[4])
    assert_close(out[:, lin], ref[:, lin], tol[:, lin], "f32", "linear")
    a_log = wl.extra["A_log"].numpy().astype(np.float64)
    dt_bias = wl.extra["dt_bias"].numpy().astype(np.float64)
    bsl, asl = slice(offs[4], offs[5]), slice(offs[5], offs[6])
    beta, tb, _, _ = O.gate_tolerances(ref[:, bsl], tol[:, bsl], a_log, dt_bias)
    _, _, dec, td = O.gate_tolerances(ref[:, asl], tol[:, asl], a_log, dt_bias)
    assert_close(out[:, bsl], beta, tb, "f32", "sigmoid gate")
    assert_close(out[:, asl], dec, td, "f32", "decay gate")
