"""CPU oracle for the NVFP4 W4A4 linear-layer path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg may import this module.  The product path
(the HIP library and its Python binding) never calls it, and this module
imports nothing from the product.  It is plain, slow and written to be checked
against the sources by eye.

Sources (one paper, "Why Gated DeltaNet Survives 4-Bit Quantization: NVFP4
W4A4 for the Recurrent Half of a Hybrid 27B LLM", arXiv 2609.04098, as quoted
by several web pages):

* NVFP4 = 4-bit E2M1 element values with one E4M3 scale per block of 16
  elements -- evolve.pub review, "Scope & Claims"; thevalue.engineering
  article, section on the fragility myth.
* Weights *and* activations are 4-bit (W4A4) on every linear layer --
  chatpaper.ai English abstract; evolve.pub review, "Summary".
* Each module carries its own per-tensor global scale, and a fused GEMM over
  several modules must keep each module's scale (the "global-scale mismatch"
  the paper repairs) -- chatpaper.ai English abstract; evolve.pub review,
  "Key claims under review", fourth claim.
* GDN gate parameterisations: write strength through a sigmoid, decay through
  a log-space softplus/exponential -- chatpaper.ai English abstract,
  mechanism (ii); evolve.pub review, "Key claims under review", second claim.

Readings where the pages are silent (each is listed with its reason in the
design notes of this repository):

* global scale g = fl32(amax / (6 * 448)), a decode multiplier: a value is
  reconstructed as e2m1 * e4m3 * g;
* block scale s = E4M3 value nearest to the exact real amax_block / (6 g),
  ties to even code, saturating at 448, OCP "FN" E4M3 (bias 7, max 448);
* element magnitude = E2M1 value nearest to the exact real |x| / (s g), ties
  to even code, saturating at 6;
* the code's sign is the IEEE sign bit of x; two codes per byte, the even
  element in the low nibble; scales one byte per block, row-major.

Exactness of the float64 arithmetic used below: inputs are float32 (a bf16
value is a float32) or float64 values with at most 30 significant bits, so
|x| has <= 30 significant bits; s has <= 4 and g
<= 24, hence s*g (<= 28 bits) and every rounding midpoint times s*g
(<= 31 bits) are exact in float64.  A non-tie quotient therefore lies at a
relative distance >= 2**-31 from every midpoint, far above the 2**-53 error of
one float64 division, and an exact tie divides to exactly the midpoint.  So a
float64 quotient compared against the grid midpoints takes exactly the
decisions of the exact-real rule.  The same argument covers amax_b / (6 g).
"""
from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------------------
# Element and scale formats
# ---------------------------------------------------------------------------

#: E2M1 magnitudes for magnitude codes 0..7 (sign bit is bit 3 of a nibble).
#: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent field 0 is
#: subnormal (0, 0.5).  No inf/NaN.
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)

E4M3_MAX = 448.0
#: 6 * 448: the largest E2M1 magnitude times the largest E4M3 value.
GLOBAL_DENOMINATOR = 6.0 * E4M3_MAX


def e4m3_decode(byte: int) -> float:
    """Value of one OCP E4M3 'FN' byte (bias 7, no inf, 0x7F/0xFF are NaN)."""
    sign = -1.0 if byte & 0x80 else 1.0
    exp = (byte >> 3) & 0xF
    man = byte & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:
        return sign * man * 2.0 ** -9  # subnormal: 0.mmm * 2^(1-7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


#: Non-negative finite E4M3 values, indexed by byte 0x00..0x7E (increasing).
E4M3_VALUES = np.array([e4m3_decode(b) for b in range(0x7F)], dtype=np.float64)


def _round_to_grid(v: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Index of the grid value nearest to each v >= 0; ties go to the even
    index; values above the last grid value saturate to it.

    ``grid`` is increasing and its index is the format's code, so "even
    index" is "even code" (even mantissa LSB).  Decisions are exact for the
    inputs this module produces (see the module docstring).
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(~np.isfinite(v)) or np.any(v < 0):
        raise ValueError("grid rounding takes finite non-negative values")
    hi = np.searchsorted(grid, v, side="left")  # first grid value >= v
    hi = np.minimum(hi, len(grid) - 1)
    lo = np.maximum(hi - 1, 0)
    exact = grid[hi] == v
    mid = (grid[lo] + grid[hi]) / 2.0  # exact: grid values have few bits
    pick_hi = (v > mid) | ((v == mid) & (hi % 2 == 0))
    idx = np.where(exact | pick_hi, hi, lo)
    idx = np.where(v >= grid[-1], len(grid) - 1, idx)  # saturation
    return idx.astype(np.uint8)


def round_e4m3(r) -> np.ndarray:
    """E4M3 byte nearest to r >= 0: ties to even, r > 448 -> 0x7E."""
    return _round_to_grid(r, E4M3_VALUES)


def round_e2m1(y) -> np.ndarray:
    """E2M1 magnitude code (0..7) nearest to y >= 0: ties to even, y > 6 -> 7."""
    return _round_to_grid(y, E2M1_MAGNITUDES)


# ---------------------------------------------------------------------------
# Quantizer (encoding) and dequantizer
# ---------------------------------------------------------------------------

def global_scale(amax: float) -> np.float32:
    """Per-tensor global scale g = fl32(amax / 2688), one RNE rounding.

    amax is a float32 value; the float64 quotient rounded to float32 equals
    the correctly rounded float32 quotient because 53 >= 2*24 + 2.
    """
    return np.float32(float(amax) / GLOBAL_DENOMINATOR)


def quantize(x: np.ndarray, g: float | None = None):
    """NVFP4-quantize a float32 matrix x [R, K] (K % 16 == 0).

    g is None -> dynamic: the global scale comes from the whole tensor's
    amax.  Otherwise g is used as given (static / calibrated scale).

    Returns (codes uint8 [R, K/2], scales uint8 [R, K/16], g float32).
    """
    x = np.asarray(x)
    if x.dtype == np.float64:
        # Allowed when every value has <= 30 significant bits (for example
        # dequantized NVFP4 values): the exactness argument above still holds.
        m, _ = np.frexp(x)
        if not np.all(np.ldexp(m, 30) == np.rint(np.ldexp(m, 30))):
            raise ValueError("float64 input must have at most 30 significant bits")
    elif x.dtype != np.float32:
        raise TypeError("oracle quantize takes float32 values (bf16 values fit exactly)")
    if x.ndim != 2 or x.shape[1] % 16 != 0:
        raise ValueError("x must be [R, K] with K % 16 == 0")
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input is outside the quantizer's contract")
    rows, cols = x.shape
    ax = np.abs(x.astype(np.float64))

    # Step 1-2: global scale.
    if g is None:
        amax = float(ax.max()) if ax.size else 0.0
        g = global_scale(amax)
    g = np.float32(g)
    g64 = float(g)

    # Step 3: one E4M3 scale per 16-element block.
    blocks = ax.reshape(rows, cols // 16, 16)
    amax_b = blocks.max(axis=2) if ax.size else np.zeros((rows, cols // 16))
    if g64 == 0.0:
        scales = np.zeros(amax_b.shape, dtype=np.uint8)
    else:
        scales = round_e4m3(amax_b / (6.0 * g64))
    s_val = E4M3_VALUES[scales]

    # Step 4: each element onto the E2M1 grid relative to s * g.
    sg = s_val * g64  # exact in float64
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.where(sg[..., None] > 0.0, blocks / sg[..., None], 0.0)
    mag = round_e2m1(y)
    mag[np.broadcast_to(sg[..., None] == 0.0, mag.shape)] = 0

    # Step 5: sign bit and nibble packing (even element -> low nibble).
    sign = np.signbit(x).reshape(rows, cols // 16, 16).astype(np.uint8)
    code = (sign << 3) | mag
    code = code.reshape(rows, cols)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, scales.astype(np.uint8), g


def unpack_codes(codes: np.ndarray, cols: int) -> np.ndarray:
    """uint8 [R, K/2] -> per-element 4-bit codes uint8 [R, K]."""
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty((codes.shape[0], cols), dtype=np.uint8)
    out[:, 0::2] = codes[:, : cols // 2] & 0xF
    out[:, 1::2] = codes[:, : cols // 2] >> 4
    return out


def dequantize(codes: np.ndarray, scales: np.ndarray, g: float, cols: int | None = None) -> np.ndarray:
    """Exact float64 values +-e2m1 * e4m3 * g of an NVFP4 matrix."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    if cols is None:
        cols = codes.shape[1] * 2
    if np.any(scales[:, : cols // 16] > 0x7E):
        raise ValueError("scale bytes must be non-negative finite E4M3 (0x00..0x7E)")
    c = unpack_codes(codes, cols)
    mag = E2M1_MAGNITUDES[c & 7]
    sign = np.where(c & 8, -1.0, 1.0)
    s = np.repeat(E4M3_VALUES[scales[:, : cols // 16]], 16, axis=1)
    return sign * mag * s * float(np.float32(g))


def storage_bytes(rows: int, cols: int) -> int:
    """Bytes of one NVFP4 tensor: half a byte per code, one byte per 16
    codes, one float32 global scale."""
    return rows * cols // 2 + rows * cols // 16 + 4


# ---------------------------------------------------------------------------
# GEMM on dequantized operands
# ---------------------------------------------------------------------------

GEMM_REL_TOL = 1e-5


def gemm(a_codes, a_scales, a_g, w_codes, w_scales, w_g, cols: int):
    """out = dec(A) @ dec(W)^T in float64, with the per-element tolerance
    T[m, n] = 1e-5 * sum_k |a[m,k] * w[n,k]|.

    Returns (ref float64 [M, N], tol float64 [M, N]).
    """
    va = dequantize(a_codes, a_scales, a_g, cols)
    vw = dequantize(w_codes, w_scales, w_g, cols)
    ref = va @ vw.T
    tol = GEMM_REL_TOL * (np.abs(va) @ np.abs(vw).T)
    return ref, tol


def dequantize_segments(w_codes, w_scales, seg_offsets, seg_g, cols: int) -> np.ndarray:
    """Dequantize a weight made of row segments, each with its own global
    scale (the per-module scales a fused GEMM has to keep)."""
    seg_offsets = [int(o) for o in seg_offsets]
    if seg_offsets[0] != 0 or any(b <= a for a, b in zip(seg_offsets, seg_offsets[1:])):
        raise ValueError("segment offsets must start at 0 and increase strictly")
    parts = []
    for s in range(len(seg_offsets) - 1):
        r0, r1 = seg_offsets[s], seg_offsets[s + 1]
        parts.append(dequantize(w_codes[r0:r1], w_scales[r0:r1], seg_g[s], cols))
    return np.concatenate(parts, axis=0)


def fused_segments(a_codes, a_scales, a_g, w_codes, w_scales, seg_offsets, seg_g, cols: int,
                   with_tol: bool = True):
    """Fused multi-module GEMM: column n of the output uses the global scale
    of the segment that holds weight row n.  Equal, by definition, to the
    concatenation of one GEMM per segment.  Returns (ref, tol); tol is None
    when with_tol is False."""
    va = dequantize(a_codes, a_scales, a_g, cols)
    vw = dequantize_segments(w_codes, w_scales, seg_offsets, seg_g, cols)
    ref = va @ vw.T
    if not with_tol:
        return ref, None
    return ref, GEMM_REL_TOL * (np.abs(va) @ np.abs(vw).T)


# ---------------------------------------------------------------------------
# Epilogue nonlinearities
# ---------------------------------------------------------------------------

def sigmoid(x) -> np.ndarray:
    """Write-strength gate beta = 1 / (1 + e^-x), float64, overflow-free."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def softplus(z) -> np.ndarray:
    """log(1 + e^z) = max(z, 0) + log1p(e^-|z|), float64."""
    z = np.asarray(z, dtype=np.float64)
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def decay_gate(x, a_log, dt_bias) -> np.ndarray:
    """Log-space decay gate -exp(A_log[h]) * softplus(x + dt_bias[h]); the
    head h is the column inside the decay segment (last axis of x)."""
    a_log = np.asarray(a_log, dtype=np.float64)
    dt_bias = np.asarray(dt_bias, dtype=np.float64)
    return -np.exp(a_log) * softplus(np.asarray(x, dtype=np.float64) + dt_bias)


def gate_tolerances(x_ref, x_tol, a_log, dt_bias):
    """Tolerances for the two gates evaluated at a pre-activation known to
    within x_tol of x_ref: |d sigmoid| <= 1/4, |d decay/dx| = exp(A_log) *
    sigmoid(x + dt_bias) (taken at the upper end of the interval, sigmoid is
    increasing), plus 2^-20 relative for the float32 evaluation."""
    x_ref = np.asarray(x_ref, dtype=np.float64)
    x_tol = np.asarray(x_tol, dtype=np.float64)
    beta = sigmoid(x_ref)
    t_beta = 0.25 * x_tol + 2.0 ** -20 * np.abs(beta)
    dec = decay_gate(x_ref, a_log, dt_bias)
    slope = np.exp(np.asarray(a_log, dtype=np.float64)) * sigmoid(x_ref + x_tol + np.asarray(dt_bias, dtype=np.float64))
    t_dec = slope * x_tol + 2.0 ** -20 * np.abs(dec)
    return beta, t_beta, dec, t_dec


# ---------------------------------------------------------------------------
# bf16 rounding, SiLU * mul glue
# ---------------------------------------------------------------------------

def round_bf16(v) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even (8
    significant bits, exponent range of float32, subnormal quantum 2^-133)."""
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("non-finite value")
    _, e = np.frexp(v)  # |v| = m * 2^e with 0.5 <= m < 1
    q = np.maximum(e - 8, -133)  # quantum of the binade (subnormal floor)
    r = np.rint(np.ldexp(v, -q))  # exact scaling, then round half even
    out = np.ldexp(r, q)
    if np.any(np.abs(out) > 3.3895313892515355e38):
        raise OverflowError("value outside the finite bf16 range")
    return out


def silu_mul(gate, up) -> np.ndarray:
    """h = bf16(silu(gate) * up), evaluated in float64 then rounded once."""
    u = np.asarray(gate, dtype=np.float64)
    w = np.asarray(up, dtype=np.float64)
    return round_bf16(u * sigmoid(u) * w)


def output_tolerance(ref, tol, out_dtype: str):
    """Allowed |out - ref| for an output stored as float32 or bf16 (bf16 adds
    half an ulp of the rounded value and an absolute floor of 2^-133)."""
    ref = np.asarray(ref, dtype=np.float64)
    tol = np.asarray(tol, dtype=np.float64)
    if out_dtype == "f32":
        return tol
    if out_dtype == "bf16":
        return tol + 2.0 ** -8 * (np.abs(ref) + tol) + 2.0 ** -133
    raise ValueError(out_dtype)


# ---------------------------------------------------------------------------
# FP8 (E4M3) KV cache with a calibrated per-tensor scale
# ---------------------------------------------------------------------------
# Sources: evolve.pub review, "Key claims under review", fifth claim
# (calibrated per-tensor FP8 KV-cache scales cost no throughput and recover
# most of FP8 KV's long-context loss); chatpaper.ai English abstract (the
# same claim).  Readings (the pages give no formula): the per-tensor scale s
# is a float32 decode multiplier (value = e4m3 * s); calibration sets
# s = fl32(amax / 448); a value x is stored as the E4M3 byte nearest to the
# exact real x / s, ties to even code, saturating at +-448, sign = IEEE sign
# bit of x; s = 1 is the uncalibrated cache.  Reading back gives
# fl32(e4m3 * s) (one rounding of the exact product); a bf16 reader rounds
# that float32 value to bf16.
#
# Exactness: x is float32 (<= 24 significant bits) and s float32, an E4M3
# midpoint has <= 5 bits, so midpoint * s (<= 29 bits) is an exact float64
# number; a non-tie x / s lies >= ~2^-28 (relative) from every midpoint, far
# above the 2^-53 error of one float64 division, and a tie divides exactly.

def kv_fp8_scale(amax) -> np.float32:
    """Calibrated per-tensor scale fl32(amax / 448), one RNE rounding."""
    return np.float32(float(np.float32(amax)) / E4M3_MAX)


def kv_fp8_quantize(x, s) -> np.ndarray:
    """E4M3 bytes of float32 values x with the per-tensor scale s > 0."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    s64 = float(np.float32(s))
    if not (s64 > 0.0 and math.isfinite(s64)):
        raise ValueError("the scale must be a positive finite float32")
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input")
    mag = round_e4m3(np.abs(x) / s64)
    sign = (np.signbit(x).astype(np.uint8) << 7).astype(np.uint8)
    return (mag | sign).astype(np.uint8)


def kv_fp8_dequantize(q, s, out_dtype: str = "f32") -> np.ndarray:
    """Values of E4M3 bytes q times s: float32 fl32(e4m3 * s), or that value
    rounded to bf16 (returned as float64 holding the bf16 value)."""
    q = np.asarray(q, dtype=np.uint8)
    if np.any((q & 0x7F) == 0x7F):
        raise ValueError("NaN code")
    mag = E4M3_VALUES[q & 0x7F]
    v = np.where(q & 0x80, -mag, mag)
    prod = (v * float(np.float32(s))).astype(np.float32)  # exact in float64, one rounding
    if out_dtype == "f32":
        return prod
    if out_dtype == "bf16":
        return round_bf16(prod.astype(np.float64))
    raise ValueError(out_dtype)


# ---------------------------------------------------------------------------
# Checkpoint-side scale harmonization of fused modules
# ---------------------------------------------------------------------------
# Sources: evolve.pub review, "Key claims under review", fourth claim (per-
# module NVFP4 calibration served by fused GEMMs corrupts the GDN gates; a
# checkpoint-side scale harmonization repairs it); chatpaper.ai English
# abstract (the global-scale mismatch of fused modules).  Readings (the pages
# give no procedure): the modules fused into one GEMM share the common global
# scale G = max_s g_s (the scale their concatenation would get, since fl32
# rounding is monotone in amax); every block scale of segment s is rewritten
# to the E4M3 value nearest to the exact real e4m3(b) * g_s / G (ties to the
# even code; the ratio is <= 1, so nothing saturates); E2M1 codes are kept.
# A kernel that applies one global scale per weight then serves the group up
# to that scale rounding; serving the per-module checkpoint with one module's
# scale is the mismatch.
#
# Exactness: e4m3(b) * g_s has <= 28 significant bits (exact in float64) and
# G has 24; a non-tie quotient lies >= ~2^-30 (relative) from every E4M3
# midpoint, and a tie divides exactly, so rounding the float64 quotient takes
# the exact-real decision.

def harmonized_global_scale(seg_g) -> np.float32:
    """Common global scale of a fused group: the largest module scale."""
    return np.float32(max(float(np.float32(g)) for g in seg_g))


def harmonize_scales(w_scales, seg_offsets, seg_g):
    """Block scales of a segmented NVFP4 weight rewritten for the common
    global scale G.  Returns (scales uint8 [N, K/16], G float32)."""
    w_scales = np.asarray(w_scales, dtype=np.uint8)
    if np.any(w_scales > 0x7E):
        raise ValueError("scale bytes must be non-negative finite E4M3 (0x00..0x7E)")
    G = harmonized_global_scale(seg_g)
    seg_offsets = [int(o) for o in seg_offsets]
    out = np.empty_like(w_scales)
    for s in range(len(seg_offsets) - 1):
        r0, r1 = seg_offsets[s], seg_offsets[s + 1]
        ratio_num = E4M3_VALUES[w_scales[r0:r1]] * float(np.float32(seg_g[s]))  # exact
        out[r0:r1] = round_e4m3(ratio_num / float(G))
    return out, G


# ---------------------------------------------------------------------------
# Gated delta-rule recurrence (the GDN state update consuming beta and g)
# ---------------------------------------------------------------------------
# Sources: chatpaper.ai English abstract, mechanism (iii) (state errors
# stay bounded and a perturbation of the state fades, since every write
# replaces what the state held along the incoming key) and mechanism (ii)
# (sigmoid write strength, log-space softplus/exponential decay); evolve.pub
# review, "Key claims under review", third claim and "Strengths" (relS
# plateau, impulse erasure).  The pages name Gated DeltaNet without writing
# out its update; the update used here is the published gated delta rule,
# per value head h with state S in R^{dv x dk}:
#
#     S_t = exp(g_t) * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
#     o_t = S_t q_t
#
# beta_t = sigmoid(b-gate), g_t = -exp(A_log) * softplus(a-gate + dt_bias)
# (the gate epilogue's outputs, a log-space decay <= 0).  Readings: q and k
# heads are shared by groups of value heads (value head h reads q/k head
# h // (Hv / Hk)); with normalize=True q and k are L2-normalized over the
# head dimension first and q is scaled by dk^-1/2, the query scale of the
# published layer (a convention of that layer, not a number the pages give;
# the short convolution that precedes q and k in a GDN layer is outside
# this path).

def l2_normalize(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, 1e-30)


def gdn_recurrence(q, k, v, beta, g, s0=None, normalize: bool = True):
    """Sequential gated delta rule in float64.

    q, k: [T, Hk, dk]; v: [T, Hv, dv]; beta, g: [T, Hv]; s0: [Hv, dv, dk] or
    None (zeros).  Returns (o [T, Hv, dv], s_final [Hv, dv, dk])."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    T, hk, dk = k.shape
    hv, dv = v.shape[1], v.shape[2]
    if hv % hk != 0:
        raise ValueError("value heads must be a multiple of key heads")
    if normalize:
        q = l2_normalize(q) / math.sqrt(dk)
        k = l2_normalize(k)
    rep = hv // hk
    qh = np.repeat(q, rep, axis=1)  # [T, Hv, dk]
    kh = np.repeat(k, rep, axis=1)
    s = np.zeros((hv, dv, dk)) if s0 is None else np.array(s0, dtype=np.float64)
    o = np.empty((T, hv, dv))
    for t in range(T):
        kt, qt = kh[t], qh[t]                      # [Hv, dk]
        a = np.exp(g[t])[:, None, None]            # decay factor
        b = beta[t][:, None]                       # [Hv, 1]
        sk = np.einsum("hij,hj->hi", s, kt)        # S_{t-1} k_t
        s = a * s - (a[:, :, 0] * b * sk)[:, :, None] * kt[:, None, :] + (b * v[t])[:, :, None] * kt[:, None, :]
        o[t] = np.einsum("hij,hj->hi", s, qt)
    return o, s
