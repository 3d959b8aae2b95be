"""GPU parity of the decode path: a weight packed into the decode layout,
the GEMM on it (nvfp4_gemm_decode) and the whole linear layer with the
activations quantized inside the launch (nvfp4_linear_decode), through the
C ABI, against the oracle on the same quantized operands (|err| <= 1e-5 *
sum|a*w| per element, plus half a bf16 ulp for bf16 output); the in-launch
quantization bit for bit against nvfp4_quantize."""
import numpy as np
import pytest
import torch

import bit_linear_layer_amd as nv
import workloads as W
from oracle import nvfp4_oracle as O
from tests.gpu_util import DEV, assert_close, host_q, oracle_weight, quantize_dev, say, weight_segments

pytestmark = pytest.mark.gpu


def rand_bf16(seed, rows, cols, scale=1.0, outliers=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)) * scale
    if outliers:
        x[:, rng.choice(cols, outliers, replace=False)] *= 50
    return W.to_bf16(x).to(DEV)


def oracle_out(a, wq, offs, seg_g):
    ac, as_, ag = host_q(a)
    wc, wsc, wg = oracle_weight(wq, offs, seg_g)
    return O.fused_segments(ac, as_, ag, wc, wsc, offs, wg, a.cols)


# (m, n, k): K slices of every chunk count 1..8 (K up to 8192), ragged K
# (16 valid elements in a lane's last chunk), ragged N (a partial 16-row
# group), one group per workgroup and many rounds per workgroup
SHAPES = [(1, 16, 16), (8, 40, 48), (3, 130, 1040), (16, 96, 2064), (8, 300, 3088), (5, 64, 4096),
          (8, 520, 5120), (2, 77, 6160), (8, 48, 7184), (16, 32, 8192), (2, 81920, 256)]


@pytest.mark.parametrize("m,n,k", SHAPES, ids=lambda v: str(v))
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_gemm_decode_shapes(m, n, k, out_dtype):
    say(f"gemm_decode {m}x{n}x{k} {out_dtype}")
    x = rand_bf16(m * 7 + n, m, k, outliers=min(2, k // 16))
    w = rand_bf16(n * 3 + k, n, k, 0.02)
    a = quantize_dev(x)
    half = max(16, (n // 2) // 16 * 16) if n > 16 else n
    offs = [0, half, n] if half < n else [0, n]
    wq, offs, seg_g = weight_segments([(str(i), w[offs[i]:offs[i + 1]]) for i in range(len(offs) - 1)])
    pw = nv.pack_decode(wq)
    dt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    out = nv.gemm_decode(a, pw, offs, seg_g, out_dtype=dt)
    ref, tol = oracle_out(a, wq, offs, seg_g)
    assert_close(out, ref, tol, out_dtype, "gemm_decode")
    # the fused in-launch quantization: same codes, same output bits
    gx = torch.empty(1, dtype=torch.float32, device=DEV)
    out2 = nv.linear_decode(x, pw, offs, seg_g, out_dtype=dt, x_global_scale=gx)
    torch.cuda.synchronize()
    assert gx.cpu().numpy().view(np.uint32)[0] == a.global_scale.cpu().numpy().view(np.uint32)[0]
    assert torch.equal(out.view(torch.int16 if out_dtype == "bf16" else torch.int32),
                       out2.view(torch.int16 if out_dtype == "bf16" else torch.int32))


@pytest.mark.parametrize("m", [1, 8, 16])
def test_linear_decode_float32_input(m):
    say(f"linear_decode float32 x, {m} rows")
    k, n = 5120, 256
    rng = np.random.default_rng(m)
    xf = torch.from_numpy((rng.standard_normal((m, k)) * 3).astype(np.float32)).to(DEV)
    w = rand_bf16(11, n, k, 0.02)
    wq, offs, seg_g = weight_segments([("w", w)])
    pw = nv.pack_decode(wq)
    a = quantize_dev(xf)
    ref = nv.gemm_decode(a, pw, offs, seg_g, out_dtype=torch.float32)
    out = nv.linear_decode(xf, pw, offs, seg_g, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.int32), out.view(torch.int32))
    r, tol = oracle_out(a, wq, offs, seg_g)
    assert_close(out, r, tol, "f32", "linear_decode f32")


def test_decode_gates_and_segments():
    """Six segments with the GDN gate epilogue on the b and a columns."""
    say("gemm_decode with gates")
    k = 5120
    sizes, sig = [64, 64, 128, 128, 48, 48], [0.01, 0.02, 0.03, 0.04, 0.05, 0.01]
    segs = [(str(i), rand_bf16(40 + i, s, k, sg)) for i, (s, sg) in enumerate(zip(sizes, sig))]
    wq, offs, seg_g = weight_segments(segs)
    x = rand_bf16(3, 8, k, outliers=2)
    a = quantize_dev(x)
    rng = np.random.default_rng(0)
    a_log = np.log(rng.uniform(1, 16, 48)).astype(np.float32)
    dt_bias = np.log(np.expm1(np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), 48)))).astype(np.float32)
    gate = dict(b_segment=4, a_segment=5, A_log=torch.from_numpy(a_log).to(DEV),
                dt_bias=torch.from_numpy(dt_bias).to(DEV))
    pw = nv.pack_decode(wq)
    out = nv.gemm_decode(a, pw, offs, seg_g, gate=gate, out_dtype=torch.float32)
    ref, tol = oracle_out(a, wq, offs, seg_g)
    o = out.cpu().numpy().astype(np.float64)
    b0, a0 = offs[4], offs[5]
    assert_close(out[:, :b0], ref[:, :b0], tol[:, :b0], "f32", "plain columns")
    beta, tb, _, _ = O.gate_tolerances(ref[:, b0:a0], tol[:, b0:a0], a_log, dt_bias)
    _, _, dec, td = O.gate_tolerances(ref[:, a0:], tol[:, a0:], a_log, dt_bias)
    assert np.all(np.abs(o[:, b0:a0] - beta) <= tb)
    assert np.all(np.abs(o[:, a0:] - dec) <= td)
    out2 = nv.linear_decode(x, pw, offs, seg_g, gate=gate, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), out2.view(torch.int32))


def test_decode_full_size_workload():
    """The 8-token decode workload: 8 x 34816 x 5120 (gate|up, two
    segments), every output element against the oracle, the linear layer
    bit-identical, and two runs bit-identical."""
    say("gemm_decode 8x34816x5120 full")
    wl = W.decode()
    wq, offs, seg_g = weight_segments(wl.weights)
    pw = nv.pack_decode(wq)
    x = wl.x.to(DEV)
    a = quantize_dev(x)
    out = nv.gemm_decode(a, pw, offs, seg_g)
    out_b = nv.gemm_decode(a, pw, offs, seg_g)
    out2 = nv.linear_decode(x, pw, offs, seg_g)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_b.view(torch.int16))
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    ref, tol = oracle_out(a, wq, offs, seg_g)
    assert_close(out, ref, tol, "bf16", "decode full size")


def test_pack_zero_pads_and_canaries():
    """The packed buffer past its size is never written, and an output with
    a wider row stride keeps its canaries."""
    say("decode pack canaries")
    m, n, k = 8, 50, 1040
    w = rand_bf16(5, n, k, 0.02)
    wq, offs, seg_g = weight_segments([("w", w)])
    nbytes = nv.nvfp4_decode_weight_bytes(n, k)
    buf = torch.full((nbytes + 4096,), 0x5A, dtype=torch.uint8, device=DEV)
    nv.nvfp4_decode_weight_pack(wq, buf[:nbytes])
    pw = nv.DecodeWeight(buf[:nbytes], n, k)
    a = quantize_dev(rand_bf16(6, m, k))
    big = torch.full((m, n + 24), 7.0, dtype=torch.float32, device=DEV)
    nv.nvfp4_gemm_decode(a, pw, offs, seg_g, big[:, :n])
    torch.cuda.synchronize()
    assert bool((buf[nbytes:] == 0x5A).all())
    assert bool((big[:, n:] == 7.0).all())
    ref, tol = oracle_out(a, wq, offs, seg_g)
    assert_close(big[:, :n], ref, tol, "f32", "decode strided out")
