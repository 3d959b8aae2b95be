"""Pins of the oracle's checkpoint-side scale harmonization (fused modules
under one common global scale) against an exact-rational nearest search,
closed forms, and the mismatch it repairs, reproduced on synthetic data
through the oracle's own GEMM."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import nvfp4_oracle as O
from tests.bruteforce import nearest_e4m3_byte

E4M3_TORCH = torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def brute_harmonize(scales, offs, seg_g):
    G = max(Fraction(float(np.float32(g))) for g in seg_g)
    out = np.empty_like(scales)
    for s in range(len(offs) - 1):
        gs = Fraction(float(np.float32(seg_g[s])))
        for idx in np.ndindex(scales[offs[s]:offs[s + 1]].shape):
            r, c = idx[0] + offs[s], idx[1]
            out[r, c] = nearest_e4m3_byte(Fraction(float(E4M3_TORCH[scales[r, c]])) * gs / G)
    return out


def test_against_exact_rational_search():
    rng = np.random.default_rng(0)
    offs = [0, 3, 5, 9]
    scales = rng.integers(0, 0x7F, size=(9, 6)).astype(np.uint8)
    seg_g = [np.float32(rng.uniform(1e-4, 1e-2)) for _ in range(3)]
    seg_g[1] = np.float32(seg_g[0] * 0.015625)  # one power-of-two ratio
    got, G = O.harmonize_scales(scales, offs, seg_g)
    assert G == max(seg_g)
    assert np.array_equal(got, brute_harmonize(scales, offs, seg_g))


def test_identity_and_top_segment_unchanged():
    rng = np.random.default_rng(1)
    scales = rng.integers(0, 0x7F, size=(12, 4)).astype(np.uint8)
    same, G = O.harmonize_scales(scales, [0, 5, 12], [np.float32(0.003)] * 2)
    assert np.array_equal(same, scales) and G == np.float32(0.003)
    out, G = O.harmonize_scales(scales, [0, 5, 12], [np.float32(0.001), np.float32(0.004)])
    assert G == np.float32(0.004)
    assert np.array_equal(out[5:], scales[5:])


def test_power_of_two_ratio_shifts_the_exponent():
    b = np.arange(0x20, 0x7F, dtype=np.uint8).reshape(-1, 1)  # normal scales, exponent >= 4
    for k in (1, 2, 3):
        out, _ = O.harmonize_scales(np.vstack([b, b]), [0, len(b), 2 * len(b)],
                                    [np.float32(2.0 ** -k), np.float32(1.0)])
        assert np.array_equal(out[:len(b), 0], b[:, 0] - 8 * k)


def test_scale_rounding_error_bound():
    rng = np.random.default_rng(2)
    scales = rng.integers(0, 0x7F, size=(40, 16)).astype(np.uint8)
    offs = [0, 10, 25, 40]
    seg_g = [np.float32(v) for v in (0.0021, 0.0007, 0.0163)]
    out, G = O.harmonize_scales(scales, offs, seg_g)
    for s in range(3):
        old = E4M3_TORCH[scales[offs[s]:offs[s + 1]]] * float(seg_g[s])
        new = E4M3_TORCH[out[offs[s]:offs[s + 1]]] * float(G)
        # half an E4M3 step: 2^-4 relative for normal results, 2^-10 absolute (times G) below
        bound = np.maximum(2.0 ** -4 * old, 2.0 ** -10 * float(G))
        assert np.all(np.abs(new - old) <= bound * (1 + 1e-12))


def gdn_like(rng, m=24, k=256):
    """Small in-projection: 6 modules with their own scales (as q/k/v/z/b/a)."""
    x = rng.standard_t(3, size=(m, k)).astype(np.float32)
    rows = [16, 16, 32, 32, 8, 8]
    sig = [0.01, 0.02, 0.03, 0.04, 0.05, 0.01]
    ws = [(rng.standard_normal((r, k)) * s).astype(np.float32) for r, s in zip(rows, sig)]
    a = O.quantize(x)
    parts = [O.quantize(w) for w in ws]
    offs = np.concatenate([[0], np.cumsum(rows)]).tolist()
    wc = np.concatenate([p[0] for p in parts])
    wsc = np.concatenate([p[1] for p in parts])
    seg_g = [p[2] for p in parts]
    return a, wc, wsc, offs, seg_g


def rel_err(x, ref):
    return float(np.linalg.norm(x - ref) / np.linalg.norm(ref))


def test_mismatch_reproduced_and_repaired():
    rng = np.random.default_rng(3)
    (ac, as_, ag), wc, wsc, offs, seg_g = gdn_like(rng)
    k = 256
    ref, _ = O.fused_segments(ac, as_, ag, wc, wsc, offs, seg_g, k, with_tol=False)
    # the mismatch: one module's scale (the first) served for every column
    bad, _ = O.gemm(ac, as_, ag, wc, wsc, seg_g[0], k)
    hs, G = O.harmonize_scales(wsc, offs, seg_g)
    fixed, _ = O.gemm(ac, as_, ag, wc, hs, G, k)
    for s in range(6):
        cols = slice(offs[s], offs[s + 1])
        ratio = float(seg_g[0]) / float(seg_g[s])
        assert rel_err(bad[:, cols], ref[:, cols]) == pytest.approx(abs(ratio - 1.0), rel=1e-9, abs=1e-12)
        assert rel_err(fixed[:, cols], ref[:, cols]) <= 2.0 ** -4
    # the gates the mismatch corrupts: beta = sigmoid on the b module
    b = slice(offs[4], offs[5])
    assert rel_err(O.sigmoid(fixed[:, b]), O.sigmoid(ref[:, b])) < 0.02
    assert rel_err(O.sigmoid(bad[:, b]), O.sigmoid(ref[:, b])) > 0.05


def test_planted_mistakes_fail():
    rng = np.random.default_rng(4)
    scales = rng.integers(8, 0x7F, size=(6, 8)).astype(np.uint8)
    offs, seg_g = [0, 3, 6], [np.float32(0.0013), np.float32(0.0101)]
    brute = brute_harmonize(scales, offs, seg_g)
    G = float(max(seg_g))
    inverted = scales.copy()
    inverted[:3] = O.round_e4m3(np.minimum(O.E4M3_VALUES[scales[:3]] * G / float(seg_g[0]), 448.0))
    assert not np.array_equal(inverted, brute)
    trunc = scales.copy()  # truncation toward zero instead of nearest
    r = O.E4M3_VALUES[scales[:3]] * float(seg_g[0]) / G
    trunc[:3] = np.searchsorted(O.E4M3_VALUES, r, side="right") - 1
    assert not np.array_equal(trunc, brute)
