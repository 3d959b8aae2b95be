"""Seeded synthetic inputs for the NVFP4 W4A4 linear-layer workloads.

Shared by the tests, the benchmark and the smoke check.  This module holds
no part of the method's arithmetic: it only draws random numbers and rounds
them to bf16 (float64 draw -> float32 -> bf16, round-to-nearest-even each
step) or float32.  Every workload uses ``numpy.random.default_rng(seed)``
with a fixed draw order: X, outlier channel ids, weight segments in order,
then the gate parameters.

Shapes and value distributions follow the paper's setting (a 5120-wide
hybrid GDN/attention model; outlier-laden residual-stream activations; a
32K-token prefill as the timed workload) -- see the design notes for the
recipe and the readings behind it.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


def to_bf16(a: np.ndarray) -> torch.Tensor:
    """float64/float32 numpy array -> bf16 CPU tensor (RNE via float32)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def bf16_to_f32_numpy(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> float32 numpy array holding the same values exactly."""
    return t.detach().to("cpu").to(torch.float32).numpy()


def outlier_activations(rng, rows: int, cols: int, *, heavy: bool, n_outlier: int, factor: float) -> np.ndarray:
    """Activations with a few large channels (residual-stream outliers).

    heavy=True draws Student-t with 3 degrees of freedom, else N(0, 1); then
    ``n_outlier`` distinct channels (columns) are multiplied by ``factor``.
    """
    if heavy:
        x = rng.standard_t(3.0, size=(rows, cols))
    else:
        x = rng.standard_normal(size=(rows, cols))
    ch = rng.choice(cols, size=n_outlier, replace=False)
    x[:, ch] *= factor
    return x


def normal_weight(rng, rows: int, cols: int, sigma: float) -> np.ndarray:
    return rng.normal(0.0, sigma, size=(rows, cols))


@dataclass
class Workload:
    name: str
    x: torch.Tensor  # bf16 [M, K]
    weights: list  # list of (name, bf16 [N_s, K]) segments, concatenated along N
    out_dtype: str = "bf16"
    extra: dict = field(default_factory=dict)

    @property
    def seg_offsets(self):
        offs = [0]
        for _, w in self.weights:
            offs.append(offs[-1] + w.shape[0])
        return offs

    def w_concat(self) -> torch.Tensor:
        return torch.cat([w for _, w in self.weights], dim=0)


def tiny(seed: int = 0, m: int = 32, n: int = 128, k: int = 256) -> Workload:
    """32x128x256 W4A4 linear, fp32 output: X ~ N(0,1) with 2 channels x50,
    W ~ N(0, 0.02)."""
    rng = np.random.default_rng(seed)
    x = outlier_activations(rng, m, k, heavy=False, n_outlier=2, factor=50.0)
    w = normal_weight(rng, n, k, 0.02)
    return Workload("tiny_m32_n128_k256", to_bf16(x), [("w", to_bf16(w))], out_dtype="f32")


def heavy_x(rng, m: int, k: int) -> np.ndarray:
    """Student-t(3) activations with 0.5% of the channels (round(0.005 K))
    scaled by 100."""
    return outlier_activations(rng, m, k, heavy=True, n_outlier=int(round(0.005 * k)), factor=100.0)


def act_quant_gemm(seed: int = 0, m: int = 4096, n: int = 5120, k: int = 5120) -> Workload:
    """Activation quantization + GEMM, bf16 output."""
    rng = np.random.default_rng(seed)
    x = heavy_x(rng, m, k)
    w = normal_weight(rng, n, k, 0.02)
    return Workload(f"act_quant_gemm_m{m}_n{n}_k{k}", to_bf16(x), [("w", to_bf16(w))])


GDN_SEGMENTS = (("q", 2048, 0.01), ("k", 2048, 0.02), ("v", 6144, 0.03),
                ("z", 6144, 0.04), ("b", 48, 0.05), ("a", 48, 0.01))


def gdn_in_proj(seed: int = 0, m: int = 32768, k: int = 5120, scale_rows: float = 1.0) -> Workload:
    """Fused GDN in-projection: six weight segments q/k/v/z/b/a, each with
    its own sigma, plus per-head A_log = ln U(1, 16) and
    dt_bias = ln(expm1(dt)), dt = exp U(ln 1e-3, ln 1e-1).

    ``scale_rows`` < 1 shrinks the four wide segments (for small test
    shapes); the two 48-row gate segments keep their width.
    """
    rng = np.random.default_rng(seed)
    x = heavy_x(rng, m, k)
    segs = []
    for name, rows, sigma in GDN_SEGMENTS:
        r = rows if rows == 48 else max(16, int(rows * scale_rows))
        segs.append((name, to_bf16(normal_weight(rng, r, k, sigma))))
    heads = 48
    a_log = np.log(rng.uniform(1.0, 16.0, size=heads)).astype(np.float32)
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=heads))
    dt_bias = np.log(np.expm1(dt)).astype(np.float32)
    name = f"gdn_in_proj_m{m}_n{sum(w.shape[0] for _, w in segs)}_k{k}"
    return Workload(name, to_bf16(x), segs,
                    extra={"A_log": torch.from_numpy(a_log), "dt_bias": torch.from_numpy(dt_bias),
                           "b_segment": 4, "a_segment": 5})


def gdn_layer(seed: int = 0, m: int = 32768, k: int = 5120) -> Workload:
    """The in-projection of one GDN layer for the recurrence study: X and the
    q/k/v/z segments as gdn_in_proj, the b and a segments scaled to the
    rows' RMS norm so that b ~ N(0, 1) and a ~ N(0, 0.25), A_log = ln U(1, 16)
    and dt_bias = inverse softplus of dt with exp(A_log) * dt = 1 / horizon,
    horizon ~ U(44000, 62000) tokens per head (the range of decay-gate
    horizons the pages report)."""
    rng = np.random.default_rng(seed)
    x = heavy_x(rng, m, k)
    xn = float(np.sqrt(np.mean(np.sum(x.astype(np.float64) ** 2, axis=1))))
    segs = []
    for name, rows, sigma in GDN_SEGMENTS:
        if name == "b":
            sigma = 1.0 / xn
        elif name == "a":
            sigma = 0.5 / xn
        segs.append((name, to_bf16(normal_weight(rng, rows, k, sigma))))
    heads = 48
    a_log = np.log(rng.uniform(1.0, 16.0, size=heads))
    horizon = rng.uniform(44000.0, 62000.0, size=heads)
    dt = 1.0 / (np.exp(a_log) * horizon)
    dt_bias = np.log(np.expm1(dt)).astype(np.float32)
    return Workload(f"gdn_layer_m{m}_k{k}", to_bf16(x), segs,
                    extra={"A_log": torch.from_numpy(a_log.astype(np.float32)),
                           "dt_bias": torch.from_numpy(dt_bias), "b_segment": 4, "a_segment": 5})


def mlp_pair(seed: int = 0, m: int = 8192, k: int = 5120, inter: int = 17408) -> Workload:
    """MLP pair: gate_up W [2*inter, k] as two segments (gate, up), then
    down W [k, inter]; all ~N(0, 0.02); heavy-tailed X."""
    rng = np.random.default_rng(seed)
    x = heavy_x(rng, m, k)
    w_gate = to_bf16(normal_weight(rng, inter, k, 0.02))
    w_up = to_bf16(normal_weight(rng, inter, k, 0.02))
    w_down = to_bf16(normal_weight(rng, k, inter, 0.02))
    return Workload(f"mlp_pair_m{m}_k{k}_i{inter}", to_bf16(x), [("gate", w_gate), ("up", w_up)],
                    extra={"w_down": w_down})


def decode(seed: int = 0, m: int = 8, k: int = 5120, inter: int = 17408) -> Workload:
    """Weight-streaming decode: M tokens x the fused gate_up weight
    [2*inter, k] (two segments); X ~ N(0,1) with 2 channels x50."""
    rng = np.random.default_rng(seed)
    x = outlier_activations(rng, m, k, heavy=False, n_outlier=2, factor=50.0)
    w_gate = to_bf16(normal_weight(rng, inter, k, 0.02))
    w_up = to_bf16(normal_weight(rng, inter, k, 0.02))
    return Workload(f"decode_m{m}_n{2 * inter}_k{k}", to_bf16(x), [("gate", w_gate), ("up", w_up)])


def kv_cache(seed: int = 0, tokens: int = 32768, heads: int = 8, head_dim: int = 128) -> Workload:
    """One layer's K tensor for the FP8 KV cache: [tokens, heads*head_dim]
    bf16, N(0,1) with 8 channels x10 (keys carry outlier channels).  The
    pages give no KV dimensions; 32K tokens is their long-context length."""
    rng = np.random.default_rng(seed)
    x = outlier_activations(rng, tokens, heads * head_dim, heavy=False, n_outlier=8, factor=10.0)
    return Workload(f"kv_cache_t{tokens}_h{heads}_d{head_dim}", to_bf16(x), [])


def random_bf16(seed: int, rows: int, cols: int, scale: float = 1.0) -> torch.Tensor:
    rng = np.random.default_rng(seed)
    return to_bf16(rng.standard_normal(size=(rows, cols)) * scale)
