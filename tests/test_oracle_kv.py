"""Pins of the oracle's FP8 (E4M3) KV-cache functions against things other
than themselves: torch's float32 -> float8_e4m3fn cast, an exact-rational
nearest search, closed forms of the calibrated scale, and invariants.  A
planted mistake (rounding a float32 quotient instead of the exact one) must
fail the brute-force pin."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import nvfp4_oracle as O

# all finite non-negative E4M3 values as exact fractions, by byte
E4M3_FRAC = [Fraction(0)] + [Fraction(m, 2 ** 9) for m in range(1, 8)] + [
    Fraction(8 + (b & 7), 8) * Fraction(2) ** ((b >> 3) - 7) for b in range(8, 0x7F)]


def brute_e4m3_byte(x: float, s: float) -> int:
    """Nearest E4M3 value to the exact real x / s by exhaustive search over
    exact fractions; ties to the even code; beyond 448 saturates."""
    r = abs(Fraction(x)) / Fraction(s)
    best = None
    for b, v in enumerate(E4M3_FRAC):
        d = abs(r - v)
        if best is None or d < best[0] or (d == best[0] and b % 2 == 0):
            best = (d, b)
    b = best[1]
    if r > E4M3_FRAC[-1]:
        b = 0x7E
    sign = 0x80 if np.signbit(np.float32(x)) else 0
    return b | sign


def test_unit_scale_matches_torch_cast_in_range():
    rng = np.random.default_rng(0)
    mids = (O.E4M3_VALUES[1:] + O.E4M3_VALUES[:-1]) / 2  # exact midpoints
    v = np.concatenate([O.E4M3_VALUES, mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                        np.nextafter(mids.astype(np.float32), np.float32(1e9)),
                        np.abs(rng.standard_normal(4000)) * 10 ** rng.uniform(-4, 2.6, 4000)])
    v = v.astype(np.float32)
    v = v[np.abs(v) <= 448]
    x = np.concatenate([v, -v])
    ours = O.kv_fp8_quantize(x, 1.0)
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_against_exact_rational_search():
    rng = np.random.default_rng(1)
    cases = []
    for _ in range(400):
        s = np.float32(10 ** rng.uniform(-3, 2))
        x = np.float32(rng.standard_normal() * s * 10 ** rng.uniform(-3, 2.8))
        cases.append((x, s))
    # exact ties: x = midpoint * s with s a power of two
    for m in ((O.E4M3_VALUES[1:] + O.E4M3_VALUES[:-1]) / 2)[::7]:
        s = np.float32(2.0 ** rng.integers(-6, 6))
        cases.append((np.float32(m * s), s))
    for x, s in cases:
        assert O.kv_fp8_quantize([x], s)[0] == brute_e4m3_byte(float(x), float(s)), (x, s)


def test_saturation_zero_and_sign():
    s = np.float32(0.5)
    assert O.kv_fp8_quantize([224.0, 232.0, 1e30, -1e30], s).tolist() == [0x7E, 0x7E, 0x7E, 0xFE]
    assert O.kv_fp8_quantize([0.0, -0.0, 2.0 ** -20], 1.0).tolist() == [0x00, 0x80, 0x00]
    x = np.random.default_rng(2).standard_normal(500).astype(np.float32)
    assert np.array_equal(O.kv_fp8_quantize(-x, 0.03), O.kv_fp8_quantize(x, 0.03) ^ 0x80)


def test_power_of_two_scale_round_trips_every_code():
    codes = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], dtype=np.uint8)
    for s in (2.0 ** -7, 1.0, 8.0):
        x = O.kv_fp8_dequantize(codes, s)
        back = O.kv_fp8_quantize(x, s)
        assert np.array_equal(back, codes)


def test_calibrated_scale_closed_form_and_range():
    rng = np.random.default_rng(3)
    x = (rng.standard_t(3, 10000) * 7).astype(np.float32)
    amax = np.abs(x).max()
    s = O.kv_fp8_scale(amax)
    assert s == np.float32(np.float64(amax) / 448.0)
    q = O.kv_fp8_quantize(x, s)
    # the largest magnitude maps to 448 (the quotient is 448 within one float32 rounding)
    assert (q[np.argmax(np.abs(x))] & 0x7F) == 0x7E
    # relative error of E4M3 with 3 mantissa bits: half a quantum, normal range
    back = O.kv_fp8_dequantize(q, s).astype(np.float64)
    normal = np.abs(x) / s >= 2.0 ** -6
    err = np.abs(back - x)[normal] / np.abs(x)[normal]
    assert err.max() <= 2.0 ** -4 * (1 + 1e-6)


def test_dequantize_matches_torch():
    codes = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], dtype=np.uint8)
    for s in (np.float32(0.0371), np.float32(3.3), np.float32(1.0)):
        f8 = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32)
        ref32 = (f8 * torch.tensor(s, dtype=torch.float32)).numpy()
        assert np.array_equal(O.kv_fp8_dequantize(codes, s), ref32)
        ref16 = torch.from_numpy(ref32).to(torch.bfloat16).to(torch.float64).numpy()
        assert np.array_equal(O.kv_fp8_dequantize(codes, s, "bf16"), ref16)


def float32_quotient_quantize(x, s):
    """A plausible mistake: round the float32 quotient x / s (two roundings)."""
    q32 = (np.asarray(x, dtype=np.float32) / np.float32(s)).astype(np.float32)
    return O.kv_fp8_quantize(q32, 1.0)


def test_planted_float32_quotient_fails_brute_force():
    # find x near an E4M3 midpoint times s whose float32 quotient lands on
    # the midpoint: the mistake then ties to even where the exact rule does not
    rng = np.random.default_rng(4)
    mids = (O.E4M3_VALUES[1:] + O.E4M3_VALUES[:-1]) / 2
    found = None
    for _ in range(20000):
        m = mids[rng.integers(8, len(mids) - 1)]
        s = np.float32(rng.uniform(0.5, 2.0))
        x = np.float32(m * float(s))
        if float(x) / float(s) == m:
            continue  # an exact tie: both rules agree
        if np.float32(x) / s != np.float32(m):
            continue
        # the float32 quotient sits on the midpoint; the mistake ties to even,
        # which is wrong when the exact quotient lies on the odd side
        if float32_quotient_quantize([x], s)[0] != brute_e4m3_byte(float(x), float(s)):
            found = (x, s)
            break
    assert found is not None
    x, s = found
    assert O.kv_fp8_quantize([x], s)[0] == brute_e4m3_byte(float(x), float(s))


@pytest.mark.parametrize("bad", [0.0, -1.0, float("inf"), float("nan")])
def test_rejects_bad_scale(bad):
    with pytest.raises(ValueError):
        O.kv_fp8_quantize([1.0], bad)
