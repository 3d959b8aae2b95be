"""Pins for the oracle's NVFP4 quantizer (CPU only).

Each test checks the oracle against something other than itself: the
bit-level format definitions, torch's float8_e4m3fn conversion, an
exact-rational brute-force quantizer, hand-worked blocks, and invariants the
format fixes.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import nvfp4_oracle as O
from tests import bruteforce as B

GOLDEN = __import__("os").path.join(__import__("os").path.dirname(__file__), "golden", "hand_worked_blocks.txt")


def f32_from_hex(h: str) -> np.float32:
    return np.array([int(h, 16)], dtype=np.uint32).view(np.float32)[0]


def f32_hex(v) -> str:
    return "0x%08X" % int(np.array([v], dtype=np.float32).view(np.uint32)[0])


def bf16_values(rng, shape, scale=1.0):
    return torch.from_numpy((rng.standard_normal(shape) * scale).astype(np.float32)).to(torch.bfloat16).float().numpy()


# --------------------------------------------------------------------- grids

def test_e2m1_grid_matches_bit_definition():
    assert [float(B.e2m1_from_bits(c)) for c in range(8)] == list(O.E2M1_MAGNITUDES)
    assert [float(B.e2m1_from_bits(c | 8)) for c in range(1, 8)] == list(-O.E2M1_MAGNITUDES[1:])


def test_e4m3_table_matches_torch_float8_e4m3fn():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(ref[:0x7F], O.E4M3_VALUES)
    assert O.E4M3_VALUES[0x38] == 1.0 and O.E4M3_VALUES[0x7E] == 448.0 and O.E4M3_VALUES[0x01] == 2.0 ** -9
    assert np.isnan(O.e4m3_decode(0x7F)) and np.isnan(O.e4m3_decode(0xFF))
    for b in range(256):
        v = O.e4m3_decode(b)
        assert (np.isnan(v) and np.isnan(ref[b])) or v == ref[b]
    assert np.all(np.diff(O.E4M3_VALUES) > 0)


def test_every_grid_value_times_every_scale_roundtrips():
    # y = m exactly for every grid value m and every nonzero scale s (static g=1)
    for sb in range(1, 0x7F):
        s = O.E4M3_VALUES[sb]
        x = np.array([[m * s for m in O.E2M1_MAGNITUDES] * 2], dtype=np.float64)
        x[0, 7] = 6 * s  # make block amax = 6 s so the scale reproduces
        x32 = x.astype(np.float32)
        if not np.array_equal(x32.astype(np.float64), x):
            continue  # value not float32-exact (never happens: <= 6 bits)
        codes, scales, _ = O.quantize(x32, g=np.float32(1.0))
        assert scales[0, 0] == sb
        assert np.array_equal(O.dequantize(codes, scales, 1.0), x)


# ------------------------------------------------------------ rounding rules

def midpoints(grid):
    return [(a + b) / 2 for a, b in zip(grid[:-1], grid[1:])]


def test_round_e4m3_matches_torch_cast():
    rng = np.random.default_rng(1)
    vals = list(rng.uniform(0, 448, 4000)) + list(rng.uniform(0, 2 ** -5, 2000))
    mids = midpoints(O.E4M3_VALUES)
    for m in mids:
        m32 = np.float32(m)
        vals += [m, float(np.nextafter(m32, np.float32(0))), float(np.nextafter(m32, np.float32(1e9)))]
    v32 = np.array(vals, dtype=np.float32)
    ours = O.round_e4m3(v32.astype(np.float64))
    theirs = torch.from_numpy(v32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_round_e4m3_saturates_and_flushes():
    assert O.round_e4m3(np.array([448.0, 460.0, 1e6]))[1:].tolist() == [0x7E, 0x7E]
    assert O.round_e4m3(np.array([2.0 ** -10]))[0] == 0  # exact tie -> even code 0
    assert O.round_e4m3(np.array([np.nextafter(2.0 ** -10, 1)]))[0] == 1


@pytest.mark.parametrize("grid,fn,bgrid", [
    (O.E2M1_MAGNITUDES, O.round_e2m1, B.E2M1_GRID),
    (O.E4M3_VALUES, O.round_e4m3, B.E4M3_GRID),
])
def test_rounding_matches_bruteforce_nearest(grid, fn, bgrid):
    rng = np.random.default_rng(2)
    vals = []
    for m in midpoints(grid):
        vals += [m, np.nextafter(m, 0.0), np.nextafter(m, np.inf)]
    vals += list(grid) + [grid[-1] * 1.01, grid[-1] * 3]
    vals += list(rng.uniform(0, grid[-1] * 1.1, 3000))
    vals = np.array(vals, dtype=np.float64)
    ours = fn(vals)
    for v, c in zip(vals, ours):
        assert c == B.nearest(Fraction(float(v)), bgrid), v


def test_e2m1_tie_table():
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    assert O.E2M1_MAGNITUDES[O.round_e2m1(ties)].tolist() == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    assert O.round_e2m1(np.array([6.0, 6.3, 100.0])).tolist() == [7, 7, 7]


# ------------------------------------------------------- hand-worked blocks

def load_golden():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, g, xs, g_exp, s_exp, c_exp = [p.strip() for p in line.split("|")]
            x = np.array([[float(v) for v in xs.split()]], dtype=np.float32)
            gin = None if g == "dynamic" else f32_from_hex(g)
            rows.append((name, x, gin, g_exp, int(s_exp, 16), bytes.fromhex(c_exp)))
    return rows


@pytest.mark.parametrize("case", load_golden(), ids=lambda c: c[0])
def test_hand_worked_blocks(case):
    name, x, g, g_exp, s_exp, c_exp = case
    # inputs are bf16-exact
    assert np.array_equal(torch.from_numpy(x).to(torch.bfloat16).float().numpy(), x)
    codes, scales, gout = O.quantize(x, g)
    assert f32_hex(gout) == g_exp
    assert scales[0, 0] == s_exp
    assert bytes(codes[0]) == c_exp
    bc, bs, bg = B.quantize_exact(x, g)
    assert bytes(bc[0]) == c_exp and bs[0, 0] == s_exp and f32_hex(bg) == g_exp


# ------------------------------------------------ brute force, random tiny

def tie_heavy_block(rng):
    """Values that are exact multiples of grid midpoints under a power-of-two
    global scale, so many elements land exactly on rounding midpoints."""
    base = rng.choice([0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 4.0, 5.0, 6.0], size=16)
    sign = rng.choice([-1.0, 1.0], size=16)
    s = 2.0 ** rng.integers(-6, 6)
    return (base * sign * s).astype(np.float32)


@pytest.mark.parametrize("seed", range(12))
def test_quantize_matches_bruteforce(seed):
    rng = np.random.default_rng(100 + seed)
    kind = seed % 4
    if kind == 0:
        x = bf16_values(rng, (3, 32))
    elif kind == 1:
        x = bf16_values(rng, (2, 48), scale=rng.uniform(1e-3, 1e3))
        x[:, 5] *= 64  # an outlier channel
    elif kind == 2:
        x = np.stack([np.concatenate([tie_heavy_block(rng), tie_heavy_block(rng)]) for _ in range(3)])
    else:
        x = (rng.standard_normal((2, 32)) * 10).astype(np.float32)  # full float32 mantissas
        x[0, :16] = 0.0
        x[1, 3] = -0.0
    for g in (None, np.float32(rng.uniform(0.001, 0.1)), np.float32(2.0 ** -6)):
        oc, os_, og = O.quantize(x, g)
        bc, bs, bg = B.quantize_exact(x, g)
        assert np.array_equal(oc, bc)
        assert np.array_equal(os_, bs)
        assert f32_hex(og) == f32_hex(bg)


def test_zero_tensor_and_signed_zero():
    x = np.zeros((2, 32), dtype=np.float32)
    x[1, 1] = -0.0
    codes, scales, g = O.quantize(x)
    assert g == 0.0 and not scales.any()
    assert codes[1, 0] == 0x80 and codes[0].sum() == 0


def test_global_scale_is_nearest_float32():
    rng = np.random.default_rng(5)
    for amax in list(rng.uniform(0, 1e4, 500).astype(np.float32)) + [np.float32(6.0), np.float32(168.0)]:
        assert f32_hex(O.global_scale(amax)) == f32_hex(B.nearest_f32(Fraction(float(amax)) / 2688))


# ---------------------------------------------------------------- invariants

def rand_x(seed, rows=8, cols=64):
    rng = np.random.default_rng(seed)
    x = bf16_values(rng, (rows, cols))
    x[:, rng.integers(0, cols)] *= 50
    return x


@settings(max_examples=40, deadline=None)
@given(st.integers(0, 10 ** 6))
def test_idempotence(seed):
    x = rand_x(seed)
    codes, scales, g = O.quantize(x)
    v = O.dequantize(codes, scales, g)  # exact float64, <= 30 significant bits
    c2, s2, g2 = O.quantize(v, g)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)
    c3, s3, g3 = O.quantize(v)  # dynamic: amax reproduces, so does g
    assert g3 == g and np.array_equal(c3, codes) and np.array_equal(s3, scales)


@settings(max_examples=40, deadline=None)
@given(st.integers(0, 10 ** 6))
def test_block_max_code_and_error_bound(seed):
    x = rand_x(seed)
    codes, scales, g = O.quantize(x)
    c = O.unpack_codes(codes, x.shape[1]).reshape(x.shape[0], -1, 16)
    s_val = O.E4M3_VALUES[scales]
    normal = s_val >= 2.0 ** -6
    # a normal, unsaturated block scale makes the block's largest element code 7
    assert np.all((c & 7).max(axis=2)[normal & (s_val < 448)] == 7)
    # unsaturated elements are within half a grid gap of their value
    v = O.dequantize(codes, scales, g).reshape(c.shape)
    sg = (s_val * float(g))[..., None]
    y = np.abs(x.astype(np.float64)).reshape(c.shape) / sg
    gaps = np.array([0.5, 0.5, 0.5, 0.5, 1.0, 1.0, 2.0, 2.0])  # gap around each code
    unsat = y <= 6.0
    err = np.abs(x.astype(np.float64).reshape(c.shape) - v)
    assert np.all(err[unsat] <= (0.5 * gaps[c & 7] * np.broadcast_to(sg, c.shape))[unsat] * (1 + 1e-12))


@settings(max_examples=30, deadline=None)
@given(st.integers(0, 10 ** 6))
def test_block_locality(seed):
    """A block's bytes depend only on its own 16 values and g."""
    rng = np.random.default_rng(seed)
    x = rand_x(seed)
    codes, scales, g = O.quantize(x)
    amax = np.abs(x).max()
    y = x.copy()
    # perturb every block except row 0 / block 1, keeping the tensor amax
    keep = y[0, 16:32].copy()
    y = y * rng.uniform(0.5, 1.0, size=y.shape).astype(np.float32)
    y[0, 16:32] = keep
    y[np.unravel_index(np.argmax(np.abs(x)), x.shape)] = x.flat[np.argmax(np.abs(x))]
    assert np.abs(y).max() == amax
    c2, s2, g2 = O.quantize(y)
    assert g2 == g
    assert np.array_equal(c2[0, 8:16], codes[0, 8:16]) and s2[0, 1] == scales[0, 1]


@settings(max_examples=30, deadline=None)
@given(st.integers(0, 10 ** 6), st.integers(-8, 8))
def test_power_of_two_equivariance_and_sign_symmetry(seed, j):
    x = rand_x(seed)
    g = np.float32(np.abs(x).max() / 2688)
    codes, scales, _ = O.quantize(x, g)
    c2, s2, _ = O.quantize((x * 2.0 ** j).astype(np.float32), np.float32(g * 2.0 ** j))
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)
    cn, sn, _ = O.quantize(-x, g)
    assert np.array_equal(sn, scales)
    assert np.array_equal(cn, codes ^ 0x88)


def test_storage_bytes_formula():
    # 0.5625 bytes per element plus one float32 per tensor
    assert O.storage_bytes(34816, 5120) == 34816 * 5120 * 9 // 16 + 4
    x = rand_x(3, 4, 64)
    codes, scales, _ = O.quantize(x)
    assert codes.nbytes + scales.nbytes + 4 == O.storage_bytes(4, 64)


def test_rejects_out_of_contract():
    with pytest.raises(ValueError):
        O.quantize(np.full((1, 16), np.nan, dtype=np.float32))
    with pytest.raises(ValueError):
        O.quantize(np.ones((1, 8), dtype=np.float32))
    with pytest.raises(TypeError):
        O.quantize(np.ones((1, 16), dtype=np.float16))
    with pytest.raises(ValueError):
        O.quantize(np.full((1, 16), 1.0 + 2.0 ** -40))  # float64 beyond 30 significant bits


# ---------------------------------------------- planted mistakes must fail

def quantize_reciprocal_f32(x, g=None):
    """A plausible wrong quantizer: float32 s*g then multiply by its
    reciprocal (not the exact quotient)."""
    amax = np.abs(x).max()
    g = np.float32(amax / np.float32(2688)) if g is None else np.float32(g)
    blocks = np.abs(x).reshape(x.shape[0], -1, 16)
    s = O.round_e4m3((blocks.max(axis=2) / np.float32(6 * g)).astype(np.float64))
    sg = np.float32(O.E4M3_VALUES[s].astype(np.float32) * g)
    y = (blocks * (np.float32(1) / sg)[..., None]).astype(np.float32)
    mag = O.round_e2m1(y.astype(np.float64))
    code = ((np.signbit(x).reshape(blocks.shape).astype(np.uint8) << 3) | mag).reshape(x.shape)
    return (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8), s, g


def test_planted_reciprocal_mistake_is_caught_by_h2():
    name, x, g, g_exp, s_exp, c_exp = [c for c in load_golden() if c[0] == "H2"][0]
    codes, scales, _ = quantize_reciprocal_f32(x, g)
    assert bytes(codes[0]) != c_exp


def test_planted_nibble_swap_is_caught_by_h1():
    name, x, g, g_exp, s_exp, c_exp = [c for c in load_golden() if c[0] == "H1"][0]
    codes, _, _ = O.quantize(x, g)
    swapped = ((codes & 0xF) << 4) | (codes >> 4)
    assert bytes(swapped[0]) != c_exp


def test_planted_ties_away_mistake_is_caught_by_h4(monkeypatch):
    name, x, g, g_exp, s_exp, c_exp = [c for c in load_golden() if c[0] == "H4"][0]

    def away(y):
        y = np.asarray(y)
        idx = np.abs(O.E2M1_MAGNITUDES[None, :] - y.reshape(-1, 1))
        best = np.where(idx == idx.min(axis=1, keepdims=True), np.arange(8), -1).max(axis=1)
        return best.reshape(y.shape).astype(np.uint8)

    monkeypatch.setattr(O, "round_e2m1", away)
    codes, _, _ = O.quantize(x, g)
    assert bytes(codes[0]) != c_exp
