"""GPU parity: NVFP4 quantization through the C ABI is bit-exact with the
oracle (codes, scales and the global scale)."""
import numpy as np
import pytest
import torch

import bit_linear_layer_amd as nv
import workloads as W
from oracle import nvfp4_oracle as O
from tests.gpu_util import DEV, assert_quant_exact, host_q, quantize_dev, say
from tests.test_oracle_quantize import f32_from_hex, f32_hex, load_golden, tie_heavy_block

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("case", load_golden(), ids=lambda c: c[0])
def test_hand_worked_blocks_on_gpu(case):
    name, x, g, g_exp, s_exp, c_exp = case
    say(f"quantize hand-worked block {name}")
    xt = torch.from_numpy(x).to(torch.bfloat16).to(DEV)
    q = quantize_dev(xt, None if g is None else float(g))
    codes, scales, gg = host_q(q)
    assert f32_hex(gg) == g_exp
    assert scales[0, 0] == s_exp
    assert bytes(codes[0]) == c_exp


# up to 1024 blocks of 16 the amax pass runs inside the one-workgroup
# quantize kernel: (64, 256) is the largest such shape, (65, 256) the next
@pytest.mark.parametrize("rows,cols", [(1, 16), (3, 32), (17, 48), (64, 160), (64, 256), (65, 256), (5, 5120),
                                       (1000, 256), (33, 1040)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_random_shapes_dynamic(rows, cols, dtype):
    say(f"quantize random {rows}x{cols} {dtype}")
    rng = np.random.default_rng(rows * 7919 + cols)
    x = rng.standard_normal((rows, cols)) * 10.0 ** rng.uniform(-3, 3)
    x[:, rng.integers(0, cols)] *= 80
    xt = torch.from_numpy(x.astype(np.float32)).to(dtype).to(DEV)
    assert_quant_exact(xt, quantize_dev(xt))


@pytest.mark.parametrize("seed", range(4))
def test_tie_heavy_dynamic_and_static(seed):
    say(f"quantize tie-heavy seed {seed}")
    rng = np.random.default_rng(1000 + seed)
    x = np.stack([np.concatenate([tie_heavy_block(rng) for _ in range(8)]) for _ in range(40)])
    xt = torch.from_numpy(x).to(torch.bfloat16).to(DEV)
    assert_quant_exact(xt, quantize_dev(xt))
    for g in (1.0, 2.0 ** -5, 0.37, 3e-3):
        assert_quant_exact(xt, quantize_dev(xt, g), g=np.float32(g))


@pytest.mark.parametrize("g", [0.37109375 * 2.0 ** -8, 0.8125 * 2.0 ** -3, 3e-3])
def test_exact_and_near_midpoints_non_power_of_two_scale(g):
    """Blocks whose scale is pinned by an element 6 * s * g; the others sit
    exactly on E2M1 midpoints mu * s * g (float32-exact when g has few
    mantissa bits) or one float32 step either side of one.  Exercises the
    kernel's exact repair of near-midpoint elements, ties included."""
    say(f"quantize midpoints g={g}")
    rng = np.random.default_rng(77)
    g = np.float32(g)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    sv = O.E4M3_VALUES[rng.integers(0x20, 0x7F, size=(48, 4))]
    x = np.empty((48, 64), np.float32)
    for r in range(48):
        for b in range(4):
            t = (rng.choice(mids, 16) * sv[r, b] * float(g)).astype(np.float32)
            t = np.where(rng.random(16) < 0.5, t, np.nextafter(t, np.float32(np.inf) * rng.choice([-1, 1], 16)))
            t[rng.integers(16)] = np.float32(6.0 * sv[r, b] * float(g))
            x[r, 16 * b:16 * b + 16] = t * rng.choice([-1.0, 1.0], 16).astype(np.float32)
    xt = torch.from_numpy(x).to(DEV)
    assert_quant_exact(xt, quantize_dev(xt, float(g)), g=g)


def test_block_scale_midpoints():
    """Blocks whose amax is 6 g times an E4M3 midpoint (exactly, and one
    float32 step either side): the block scale's rounding decision itself
    sits on or next to a tie (the kernel's bracketed scale path and its
    exact repair)."""
    say("quantize block-scale midpoints")
    g = np.float32(0.8125 * 2.0 ** -5)
    vals = O.E4M3_VALUES[:0x7F]
    mids = 0.5 * (vals[:-1] + vals[1:])
    am = (6.0 * float(g) * mids).astype(np.float32)
    am = np.concatenate([am, np.nextafter(am, np.float32(np.inf)), np.nextafter(am, np.float32(0))])
    rng = np.random.default_rng(21)
    x = (rng.uniform(-1, 1, (am.size, 16)) * am[:, None]).astype(np.float32)
    x[np.arange(am.size), rng.integers(0, 16, am.size)] = am * rng.choice([-1, 1], am.size).astype(np.float32)
    x = x.reshape(-1, 64) if x.shape[0] % 4 == 0 else x[: x.shape[0] // 4 * 4].reshape(-1, 64)
    xt = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    assert_quant_exact(xt, quantize_dev(xt, float(g)), g=g)


@pytest.mark.parametrize("mag", [1e-30, 1e-39])
def test_tiny_magnitudes(mag):
    """float32 inputs so small that s * g lies below 2^-90 (the kernel's
    exact threshold count instead of its bracketed hardware pack); at 1e-39
    the inputs and the global scale are subnormal."""
    say(f"quantize tiny magnitudes {mag}")
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((8, 64)) * mag).astype(np.float32)
    xt = torch.from_numpy(x).to(DEV)
    assert_quant_exact(xt, quantize_dev(xt))
    gs = float(np.float32(mag * 0.01))
    assert_quant_exact(xt, quantize_dev(xt, gs), g=np.float32(gs))


def test_static_scale_saturation():
    """A too-small calibrated scale saturates block scales at 448 and
    elements at 6."""
    say("quantize static saturation")
    rng = np.random.default_rng(3)
    xt = torch.from_numpy(rng.standard_normal((8, 64)).astype(np.float32) * 100).to(torch.bfloat16).to(DEV)
    q = quantize_dev(xt, 1e-4)
    assert_quant_exact(xt, q, g=np.float32(1e-4))
    codes, scales, _ = host_q(q)
    assert (scales == 0x7E).mean() > 0.9


def test_zero_and_signed_zero():
    say("quantize zeros")
    x = torch.zeros((4, 32), dtype=torch.bfloat16)
    x[1, 3] = -0.0
    xt = x.to(DEV)
    q = quantize_dev(xt)
    codes, scales, g = host_q(q)
    assert g == 0 and not scales.any()
    assert codes[1, 1] == 0x80 and codes[0].sum() == 0
    assert_quant_exact(xt, q)


def test_strided_rows_and_fp32_input():
    say("quantize strided rows")
    rng = np.random.default_rng(4)
    big = torch.from_numpy(rng.standard_normal((12, 96)).astype(np.float32)).to(DEV)
    view = big[:, :64]  # ld_x = 96 > cols = 64
    assert_quant_exact(view, quantize_dev(view))


def test_activation_config_full_size_and_determinism():
    """4096x5120 Student-t activations with 0.5% outlier channels, full
    bit-exact comparison, and two runs give identical bytes."""
    say("quantize act_quant_gemm X 4096x5120")
    rng = np.random.default_rng(0)
    x = W.to_bf16(W.heavy_x(rng, 4096, 5120)).to(DEV)
    q1 = quantize_dev(x)
    assert_quant_exact(x, q1)
    q2 = quantize_dev(x)
    c1, s1, g1 = host_q(q1)
    c2, s2, g2 = host_q(q2)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2) and g1 == g2


def test_prefill_32k_sampled_rows():
    """32768x5120 activations (the 32K-token prefill): g from the whole
    tensor, codes/scales compared on 512 rows incl. the first and last."""
    say("quantize 32768x5120 sampled")
    rng = np.random.default_rng(0)
    x = W.to_bf16(W.heavy_x(rng, 32768, 5120)).to(DEV)
    q = quantize_dev(x)
    rows = np.unique(np.concatenate([[0, 1, 32767], np.random.default_rng(1).integers(0, 32768, 509)]))
    assert_quant_exact(x, q, rows=rows)
