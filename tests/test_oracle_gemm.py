"""Pins for the oracle's GEMM, fused segments, gate epilogue, bf16 rounding
and SiLU*mul glue (CPU only)."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import nvfp4_oracle as O
from tests import bruteforce as B


def bf16_np(rng, shape, scale=1.0):
    return torch.from_numpy((rng.standard_normal(shape) * scale).astype(np.float32)).to(torch.bfloat16).float().numpy()


def quantized_pair(seed, m, n, k):
    rng = np.random.default_rng(seed)
    a = O.quantize(bf16_np(rng, (m, k)))
    w = O.quantize(bf16_np(rng, (n, k), 0.02))
    return a, w


# ---------------------------------------------------------------- GEMM

@pytest.mark.parametrize("seed,m,n,k", [(0, 3, 4, 64), (1, 4, 2, 32), (2, 1, 3, 48), (3, 2, 2, 16)])
def test_gemm_matches_exact_fraction_sums(seed, m, n, k):
    (ac, as_, ag), (wc, ws, wg) = quantized_pair(seed, m, n, k)
    ref, tol = O.gemm(ac, as_, ag, wc, ws, wg, k)
    # independent decode of every element through the brute-force grids
    def dec(codes, scales, g):
        out = []
        for r in range(codes.shape[0]):
            row = []
            for j in range(k):
                byte = int(codes[r, j // 2])
                c = byte & 0xF if j % 2 == 0 else byte >> 4
                row.append(B.e2m1_from_bits(c) * B.E4M3_GRID[int(scales[r, j // 16])][0] * Fraction(float(g)))
            out.append(row)
        return out
    va, vw = dec(ac, as_, ag), dec(wc, ws, wg)
    for i in range(m):
        for j in range(n):
            exact = sum(va[i][t] * vw[j][t] for t in range(k))
            absum = sum(abs(va[i][t] * vw[j][t]) for t in range(k))
            assert abs(Fraction(float(ref[i, j])) - exact) <= Fraction(1, 10 ** 12) * absum + Fraction(1, 10 ** 300)
            assert abs(Fraction(float(tol[i, j])) - absum / 100000) <= absum * Fraction(1, 10 ** 15)


def test_gemm_one_hot_weights_select_columns():
    rng = np.random.default_rng(7)
    k = 64
    a = O.quantize(bf16_np(rng, (5, k)))
    va = O.dequantize(*a, cols=k)
    # W row n: code 2 (=1.0) at column n, 0 elsewhere; scales 0x38 (1.0); static g = 1
    n = 6
    codes = np.zeros((n, k // 2), dtype=np.uint8)
    for r in range(n):
        col = 9 * r + 1
        codes[r, col // 2] = 2 << (4 * (col % 2))
    scales = np.full((n, k // 16), 0x38, dtype=np.uint8)
    ref, tol = O.gemm(*a, codes, scales, np.float32(1.0), k)
    for r in range(n):
        assert np.array_equal(ref[:, r], va[:, 9 * r + 1])


def test_gemm_all_ones_gives_k():
    k = 96
    codes = np.full((3, k // 2), 0x22, dtype=np.uint8)  # 1.0, 1.0
    scales = np.full((3, k // 16), 0x38, dtype=np.uint8)
    ref, tol = O.gemm(codes, scales, 1.0, codes, scales, 1.0, k)
    assert np.all(ref == k) and np.allclose(tol, 1e-5 * k)


def test_gemm_operand_orientation():
    """out[m, n] pairs row m of A with row n of W (out = A W^T): a transposed
    operand or swapped roles would fail on a non-square shape."""
    (ac, as_, ag), (wc, ws, wg) = quantized_pair(11, 2, 5, 32)
    ref, _ = O.gemm(ac, as_, ag, wc, ws, wg, 32)
    assert ref.shape == (2, 5)
    va = O.dequantize(ac, as_, ag)
    vw = O.dequantize(wc, ws, wg)
    assert ref[1, 3] == pytest.approx(float(np.dot(va[1], vw[3])), rel=1e-14)


# ------------------------------------------------------------ segments

def make_segments(seed, k=64, rows=(16, 8, 24), sigmas=(0.01, 0.05, 0.2)):
    rng = np.random.default_rng(seed)
    a = O.quantize(bf16_np(rng, (4, k)))
    segs = [O.quantize(bf16_np(rng, (r, k), s)) for r, s in zip(rows, sigmas)]
    codes = np.concatenate([s[0] for s in segs])
    scales = np.concatenate([s[1] for s in segs])
    offs = np.concatenate([[0], np.cumsum(rows)])
    gs = np.array([s[2] for s in segs], dtype=np.float32)
    return a, segs, codes, scales, offs, gs


def test_fused_equals_concatenated_per_segment_gemms():
    k = 64
    a, segs, codes, scales, offs, gs = make_segments(3, k)
    fused, ftol = O.fused_segments(*a, codes, scales, offs, gs, k)
    parts = [O.gemm(*a, *s, k) for s in segs]
    assert np.array_equal(fused, np.concatenate([p[0] for p in parts], axis=1))
    assert np.array_equal(ftol, np.concatenate([p[1] for p in parts], axis=1))


def test_single_global_scale_reproduces_the_mismatch():
    """Serving the fused weight with segment 0's global scale scales segment
    s by exactly g_w[0] / g_w[s] -- the failure mode the per-segment
    epilogue avoids."""
    k = 64
    a, segs, codes, scales, offs, gs = make_segments(4, k)
    good, _ = O.fused_segments(*a, codes, scales, offs, gs, k)
    bad, _ = O.fused_segments(*a, codes, scales, offs, np.full_like(gs, gs[0]), k)
    for s in range(len(gs)):
        sl = slice(offs[s], offs[s + 1])
        ratio = float(gs[0]) / float(gs[s])
        assert np.allclose(bad[:, sl], good[:, sl] * ratio, rtol=1e-13, atol=0)
        if s > 0:
            assert not np.allclose(bad[:, sl], good[:, sl], rtol=1e-3)


def test_segment_table_validation():
    a, segs, codes, scales, offs, gs = make_segments(5)
    with pytest.raises(ValueError):
        O.fused_segments(*a, codes, scales, [0, 16, 16, 48], gs, 64)
    with pytest.raises(ValueError):
        O.fused_segments(*a, codes, scales, [1, 16, 24, 48], gs, 64)


# ----------------------------------------------------------------- gates

def test_gate_special_values():
    assert O.sigmoid(np.array([0.0]))[0] == 0.5
    a_log = np.array([0.0, np.log(3.0)])
    dt_bias = np.array([0.25, -1.5])
    x = -dt_bias  # x + dt_bias = 0 -> softplus = ln 2
    assert np.allclose(O.decay_gate(x, a_log, dt_bias), -np.exp(a_log) * np.log(2.0), rtol=1e-15)
    assert O.sigmoid(np.array([-800.0]))[0] == 0.0 and O.sigmoid(np.array([800.0]))[0] == 1.0
    assert O.softplus(np.array([800.0]))[0] == 800.0


def test_gates_match_torch_float64():
    rng = np.random.default_rng(9)
    x = rng.standard_normal(2000) * 20
    a_log = np.log(rng.uniform(1, 16, 2000))
    dt_bias = np.log(np.expm1(np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), 2000))))
    tx = torch.from_numpy(x)
    assert np.allclose(O.sigmoid(x), torch.sigmoid(tx).numpy(), rtol=1e-14, atol=1e-300)
    ref = -torch.exp(torch.from_numpy(a_log)) * torch.nn.functional.softplus(tx + torch.from_numpy(dt_bias), threshold=1e9)
    assert np.allclose(O.decay_gate(x, a_log, dt_bias), ref.numpy(), rtol=1e-13, atol=1e-300)


def test_gates_monotone():
    x = np.linspace(-30, 30, 5001)
    assert np.all(np.diff(O.sigmoid(x)) >= 0)
    assert np.all(np.diff(O.decay_gate(x, 1.0, 0.5)) <= 0)
    assert np.all(O.decay_gate(x, 1.0, 0.5) < 0)


def test_gate_tolerance_bounds_the_slope():
    rng = np.random.default_rng(10)
    x = rng.standard_normal(500) * 5
    dx = np.abs(rng.standard_normal(500)) * 1e-3
    a_log, dt_bias = 1.2, -3.0
    beta, tb, dec, td = O.gate_tolerances(x, dx, a_log, dt_bias)
    for sgn in (-1, 1):
        xs = x + sgn * dx
        assert np.all(np.abs(O.sigmoid(xs) - beta) <= tb)
        assert np.all(np.abs(O.decay_gate(xs, a_log, dt_bias) - dec) <= td)


# ----------------------------------------------------- bf16, SiLU * mul

def test_round_bf16_matches_bruteforce():
    rng = np.random.default_rng(12)
    vals = list(rng.standard_normal(400) * 10 ** rng.uniform(-30, 30, 400))
    # exact bf16 midpoints and their float64 neighbours
    for b in rng.integers(0, 0x7F00, 100):
        lo = np.array([b << 16], dtype=np.uint32).view(np.float32)[0]
        hi = np.array([(b + 1) << 16], dtype=np.uint32).view(np.float32)[0]
        mid = (float(lo) + float(hi)) / 2
        vals += [mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf), -mid]
    vals += [2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135, 0.0]
    ours = O.round_bf16(np.array(vals))
    for v, o in zip(vals, ours):
        assert o == B.bf16_nearest(Fraction(float(v))), v


def test_round_bf16_matches_torch_for_float32_inputs():
    rng = np.random.default_rng(13)
    v = (rng.standard_normal(10000) * 10 ** rng.uniform(-20, 20, 10000)).astype(np.float32)
    theirs = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_bf16(v.astype(np.float64)), theirs)


def test_silu_mul_closed_forms():
    u = np.array([0.0, 30.0, -50.0, 1.0])
    w = np.array([5.0, 2.0, 3.0, 1.0])
    h = O.silu_mul(u, w)
    assert h[0] == 0.0 and h[1] == 60.0 and h[2] == O.round_bf16(-50.0 * 3.0 * np.exp(-50.0) / (1 + np.exp(-50.0)))
    assert h[3] == O.round_bf16(1.0 / (1.0 + np.exp(-1.0)))


def test_silu_mul_matches_torch_silu():
    rng = np.random.default_rng(14)
    u = rng.standard_normal(5000) * 4
    w = rng.standard_normal(5000)
    ref = (torch.nn.functional.silu(torch.from_numpy(u)) * torch.from_numpy(w)).numpy()
    ours = O.silu_mul(u, w)
    # both evaluate in float64, so they can differ only where the float64
    # value sits on a bf16 midpoint; every result is within half a bf16 ulp
    assert np.mean(ours == O.round_bf16(ref)) > 0.999
    assert np.all(np.abs(ours - ref) <= 2.0 ** -8 * np.abs(ref) * (1 + 1e-12) + 2.0 ** -133)


def test_output_tolerance_terms():
    ref = np.array([1.0, -3.0])
    tol = np.array([1e-5, 0.0])
    assert np.array_equal(O.output_tolerance(ref, tol, "f32"), tol)
    bt = O.output_tolerance(ref, tol, "bf16")
    assert bt[0] == pytest.approx(1e-5 + 2 ** -8 * (1 + 1e-5) + 2 ** -133)
    # the bf16 term covers the rounding of any value within tol of ref
    for v in (1.0 + 1e-5, 3.0):
        assert abs(O.round_bf16(np.array([v]))[0] - v) <= 2 ** -8 * v
