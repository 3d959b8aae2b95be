"""GPU parity for the FP8 (E4M3) KV cache: calibration, the cache write
(with and without a slot scatter) and the read, bit-exact against the
oracle on ragged, tie-laden, saturating and full-size inputs."""
import numpy as np
import pytest
import torch

import bit_linear_layer_amd as nv
import workloads as W
from oracle import nvfp4_oracle as O
from tests.gpu_util import DEV, say

pytestmark = pytest.mark.gpu


def f32_cases(rng, rows, cols, s):
    """float32 values: exact ties (midpoint * s for a power-of-two s), their
    float32 neighbours, zeros of both signs, saturating values, random."""
    mids = (O.E4M3_VALUES[1:] + O.E4M3_VALUES[:-1]) / 2
    pool = np.concatenate([mids * s, O.E4M3_VALUES * s, [0.0, -0.0, 460 * s, 1e6 * s, 2.0 ** -12 * s]])
    pool = pool.astype(np.float32)
    pool = np.concatenate([pool, np.nextafter(pool, np.float32(np.inf)), np.nextafter(pool, np.float32(-np.inf))])
    x = rng.choice(pool, size=(rows, cols)) * rng.choice([-1.0, 1.0], size=(rows, cols))
    x = x.astype(np.float32)
    x[rows // 2:] = (rng.standard_normal((rows - rows // 2, cols)) * s * 40).astype(np.float32)
    return x


@pytest.mark.parametrize("rows,cols", [(1, 16), (37, 1040), (256, 128)])
@pytest.mark.parametrize("s", [1.0, 0.0625, 0.37109375])
def test_kv_write_read_float32_exact(rows, cols, s):
    say(f"kv fp8 f32 {rows}x{cols} s={s}")
    rng = np.random.default_rng(rows + cols)
    x = f32_cases(rng, rows, cols, s)
    sc = torch.tensor([s], dtype=torch.float32, device=DEV)
    cache = nv.kv_fp8_quantize(torch.from_numpy(x).to(DEV), sc)
    out32 = nv.kv_fp8_dequantize(cache, sc, torch.float32)
    out16 = nv.kv_fp8_dequantize(cache, sc, torch.bfloat16)
    torch.cuda.synchronize()
    q = O.kv_fp8_quantize(x, s)
    got = cache.cpu().numpy()
    bad = np.argwhere(got != q)
    assert bad.size == 0, f"{len(bad)} bytes differ, first {bad[:3].tolist()}"
    ref32 = O.kv_fp8_dequantize(q, s)
    assert np.array_equal(out32.cpu().numpy().view(np.uint32), ref32.view(np.uint32))
    assert np.array_equal(W.bf16_to_f32_numpy(out16).astype(np.float64), O.kv_fp8_dequantize(q, s, "bf16"))


@pytest.mark.parametrize("s", [1.0, 0.0625, 0.37109375, 3.3e-3])
@pytest.mark.parametrize("layout", ["contiguous", "strided"])
def test_kv_write_in_range_ties(s, layout):
    """Ties, their neighbours and grid values with no saturating element, so
    whole wavefronts take the write's unclamped bracket; contiguous rows run
    the linear-index kernel, strided rows the (row, chunk) walk."""
    say(f"kv fp8 in-range ties s={s} {layout}")
    rng = np.random.default_rng(17)
    rows, cols = 96, 1024
    mids = (O.E4M3_VALUES[1:] + O.E4M3_VALUES[:-1]) / 2
    pool = np.concatenate([mids * s, O.E4M3_VALUES * s, [0.0, -0.0]]).astype(np.float32)
    pool = np.concatenate([pool, np.nextafter(pool, np.float32(np.inf)), np.nextafter(pool, np.float32(-np.inf))])
    pool = pool[np.abs(pool.astype(np.float64)) / np.float64(np.float32(s)) < 447.0]
    x = (rng.choice(pool, size=(rows, cols)) * rng.choice([-1.0, 1.0], size=(rows, cols))).astype(np.float32)
    xd = torch.from_numpy(x).to(DEV)
    if layout == "strided":
        wide = torch.zeros((rows, cols + 64), dtype=torch.float32, device=DEV)
        wide[:, :cols] = xd
        xd = wide[:, :cols]
    sc = torch.tensor([s], dtype=torch.float32, device=DEV)
    cache = nv.kv_fp8_quantize(xd, sc)
    torch.cuda.synchronize()
    got = cache.cpu().numpy()
    bad = np.argwhere(got != O.kv_fp8_quantize(x, s))
    assert bad.size == 0, f"{len(bad)} bytes differ, first {bad[:3].tolist()}"


@pytest.mark.parametrize("s", [1e-40, 2.0 ** -126, 2.0 ** -120, 3.0e30])
def test_kv_write_extreme_scales(s):
    """Subnormal, smallest-normal and huge scales (the write's estimate of
    1/s overflows for subnormal s and the kernel divides instead)."""
    say(f"kv fp8 extreme scale {s}")
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((8, 64)) * 10.0 ** rng.integers(-40, 38, (8, 64))).astype(np.float32)
    x[0, :4] = [0.0, -0.0, 1e-45, -1e-45]
    s32 = np.float32(s)
    sc = torch.tensor([s32], dtype=torch.float32, device=DEV)
    cache = nv.kv_fp8_quantize(torch.from_numpy(x).to(DEV), sc)
    torch.cuda.synchronize()
    assert np.array_equal(cache.cpu().numpy(), O.kv_fp8_quantize(x, s32))


def test_kv_every_code_reads_back():
    codes = np.array([b for b in range(256) if (b & 0x7F) != 0x7F] * 2, dtype=np.uint8)[:496].reshape(31, 16)
    for s in (1.0, 0.013, 7.5):
        sc = torch.tensor([s], dtype=torch.float32, device=DEV)
        c = torch.from_numpy(codes).to(DEV)
        out32 = nv.kv_fp8_dequantize(c, sc, torch.float32)
        torch.cuda.synchronize()
        ref = O.kv_fp8_dequantize(codes, np.float32(s))
        assert np.array_equal(out32.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("rows,cols", [(300, 1024), (4096, 1024)])
def test_kv_calibrated_bf16_cache(rows, cols):
    say(f"kv fp8 calibrated bf16 {rows}x{cols}")
    rng = np.random.default_rng(cols)
    xb = W.to_bf16(W.outlier_activations(rng, rows, cols, heavy=True, n_outlier=4, factor=30.0)).to(DEV)
    s = nv.kv_fp8_calibrate(xb)
    cache = nv.kv_fp8_quantize(xb, s)
    torch.cuda.synchronize()
    xf = W.bf16_to_f32_numpy(xb)
    s_ref = O.kv_fp8_scale(np.abs(xf).max())
    assert s.cpu().numpy()[0].view(np.uint32) == np.float32(s_ref).view(np.uint32)
    q = O.kv_fp8_quantize(xf, s_ref)
    assert np.array_equal(cache.cpu().numpy(), q)
    assert ((q & 0x7F) == 0x7E).any()  # the amax lands on 448


def test_kv_slot_scatter_and_out_of_range_rows():
    say("kv fp8 slots")
    rng = np.random.default_rng(11)
    rows, cols, cache_rows = 64, 256, 200
    x = (rng.standard_normal((rows, cols)) * 3).astype(np.float32)
    slots = rng.permutation(cache_rows)[:rows].astype(np.int64)
    slots[5] = -1
    slots[9] = cache_rows  # both skipped
    sc = torch.tensor([0.02], dtype=torch.float32, device=DEV)
    cache = torch.full((cache_rows, cols), 0x5A, dtype=torch.uint8, device=DEV)
    nv.nvfp4_kv_fp8_quantize(torch.from_numpy(x).to(DEV), cache, sc, torch.from_numpy(slots).to(DEV))
    torch.cuda.synchronize()
    got = cache.cpu().numpy()
    q = O.kv_fp8_quantize(x, np.float32(0.02))
    expect = np.full((cache_rows, cols), 0x5A, dtype=np.uint8)
    ok = (slots >= 0) & (slots < cache_rows)
    expect[slots[ok]] = q[ok]
    assert np.array_equal(got, expect)


def test_kv_full_size_write_and_read():
    """32768 tokens x 1024 (8 heads x 128), bf16, calibrated: whole arrays."""
    say("kv fp8 32768x1024")
    rng = np.random.default_rng(0)
    xb = W.to_bf16(rng.standard_normal((32768, 1024)) * 2).to(DEV)
    s = nv.kv_fp8_calibrate(xb)
    cache = nv.kv_fp8_quantize(xb, s)
    back = nv.kv_fp8_dequantize(cache, s, torch.bfloat16)
    torch.cuda.synchronize()
    xf = W.bf16_to_f32_numpy(xb)
    s_ref = O.kv_fp8_scale(np.abs(xf).max())
    assert s.cpu().numpy()[0] == s_ref
    q = O.kv_fp8_quantize(xf, s_ref)
    assert np.array_equal(cache.cpu().numpy(), q)
    assert np.array_equal(W.bf16_to_f32_numpy(back).astype(np.float64), O.kv_fp8_dequantize(q, s_ref, "bf16"))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_kv_cache_rows_8_byte_aligned(dtype):
    """A cache whose rows start 8 (not 16) bytes apart: the write stores in
    8-byte halves and the read loads them the same way; the padding bytes of
    each row stay untouched, and the bytes equal those of a dense cache."""
    say(f"kv fp8 cache rows 8-byte aligned {dtype}")
    rng = np.random.default_rng(21)
    rows, cols = 333, 272
    x = torch.from_numpy((rng.standard_normal((rows, cols)) * 7).astype(np.float32)).to(dtype).to(DEV)
    sc = nv.kv_fp8_calibrate(x)
    dense = nv.kv_fp8_quantize(x, sc)
    big = torch.full((rows, cols + 8), 0xA5, dtype=torch.uint8, device=DEV)
    nv.nvfp4_kv_fp8_quantize(x, big[:, :cols], sc)
    torch.cuda.synchronize()
    assert big.stride(0) % 16 == 8
    xf = x.float().cpu().numpy()
    assert np.array_equal(dense.cpu().numpy(), O.kv_fp8_quantize(xf, np.float32(sc.cpu().numpy()[0])))
    assert torch.equal(big[:, :cols], dense)
    assert bool((big[:, cols:] == 0xA5).all())
    out_dense = nv.kv_fp8_dequantize(dense, sc, out_dtype=dtype)
    out = torch.empty((rows, cols), dtype=dtype, device=DEV)
    nv.nvfp4_kv_fp8_dequantize(big[:, :cols], sc, out, cols)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16 if dtype == torch.bfloat16 else torch.int32),
                       out_dense.view(torch.int16 if dtype == torch.bfloat16 else torch.int32))
