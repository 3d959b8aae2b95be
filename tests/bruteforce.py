"""Exact-rational brute-force NVFP4 reference for pinning the oracle.

Independent of the oracle: grids are enumerated from the bit-level format
definitions (E2M1 here, E4M3 through torch's float8_e4m3fn), every rounding
is a nearest-value search over exact fractions with ties to the even code,
and saturation falls out of the search (beyond the largest value the largest
value is nearest).  Only usable on tiny inputs.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import torch


def e2m1_from_bits(code: int) -> Fraction:
    """E2M1: 1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit."""
    sign = -1 if code & 8 else 1
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        mag = Fraction(m, 2)  # subnormal 0.m * 2^(1-1)
    else:
        mag = (1 + Fraction(m, 2)) * Fraction(2) ** (e - 1)
    return sign * mag


E2M1_GRID = [(e2m1_from_bits(c), c) for c in range(8)]

_e4m3_all = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
E4M3_GRID = [(Fraction(float(_e4m3_all[b])), b) for b in range(0x7F)]  # 0x00..0x7E


def nearest(v: Fraction, grid) -> int:
    best = None
    for val, code in grid:
        d = abs(v - val)
        key = (d, code % 2)  # smaller distance first, then even code
        if best is None or key < best[0]:
            best = (key, code)
    return best[1]


def nearest_f32(q: Fraction) -> np.float32:
    """float32 nearest to q (ties to even significand) by neighbour search."""
    c = np.float32(float(q))
    cands = {c, np.nextafter(c, np.float32(-np.inf)), np.nextafter(c, np.float32(np.inf))}
    best = None
    for f in cands:
        d = abs(Fraction(float(f)) - q)
        key = (d, int(np.array(f, dtype=np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, f)
    return np.float32(best[1])


def quantize_exact(x: np.ndarray, g=None):
    """Brute-force NVFP4 quantization of a float32 [R, K] array."""
    rows, cols = x.shape
    xs = [[Fraction(float(v)) for v in row] for row in x]
    if g is None:
        amax = max((abs(v) for row in xs for v in row), default=Fraction(0))
        g = nearest_f32(amax / (6 * 448))
    gq = Fraction(float(np.float32(g)))
    codes = np.zeros((rows, cols // 2), dtype=np.uint8)
    scales = np.zeros((rows, cols // 16), dtype=np.uint8)
    for r in range(rows):
        for j in range(cols // 16):
            blk = xs[r][16 * j:16 * j + 16]
            amax_b = max(abs(v) for v in blk)
            if gq == 0 or amax_b == 0:
                sbyte = 0
            else:
                sbyte = nearest(amax_b / (6 * gq), E4M3_GRID)
            scales[r, j] = sbyte
            sval = E4M3_GRID[sbyte][0]
            for i, v in enumerate(blk):
                if sval == 0:
                    mag = 0
                else:
                    mag = nearest(abs(v) / (sval * gq), E2M1_GRID)
                neg = np.signbit(np.float32(x[r, 16 * j + i]))
                code = (8 if neg else 0) | mag
                k = 16 * j + i
                if k % 2 == 0:
                    codes[r, k // 2] |= code
                else:
                    codes[r, k // 2] |= code << 4
    return codes, scales, np.float32(g)


def bf16_nearest(v: Fraction) -> float:
    """Nearest bf16 value to v (ties to even) by searching the neighbours of
    float32 rounding."""
    f = np.float32(float(v))
    bits = int(np.array(f, dtype=np.float32).view(np.uint32))
    base = bits & 0xFFFF0000
    cands = []
    for b in (base - 0x10000, base, base + 0x10000, base + 0x20000):
        if b < 0:
            continue
        val = np.array([b & 0xFFFFFFFF], dtype=np.uint32).view(np.float32)[0]
        if np.isfinite(val):
            cands.append((abs(Fraction(float(val)) - v), (b >> 16) & 1, float(val)))
    cands.sort()
    return cands[0][2]


def nearest_e4m3_byte(r) -> int:
    """E4M3 byte (0x00..0x7E) nearest to the exact rational r >= 0 by
    exhaustive search over all finite values built from the bit definition;
    ties to the even code; r beyond 448 saturates."""
    from fractions import Fraction
    vals = [Fraction(m, 2 ** 9) for m in range(8)] + [
        Fraction(8 + (b & 7), 8) * Fraction(2) ** ((b >> 3) - 7) for b in range(8, 0x7F)]
    r = Fraction(r)
    if r > vals[-1]:
        return 0x7E
    best = None
    for b, v in enumerate(vals):
        d = abs(r - v)
        if best is None or d < best[0] or (d == best[0] and b % 2 == 0):
            best = (d, b)
    return best[1]
