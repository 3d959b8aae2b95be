"""GPU parity for the chunked gated delta-rule recurrence against the
oracle's sequential float64 definition: ragged lengths (partial last
chunk), grouped heads, normalized and raw q/k, an initial state, bf16 and
float32 inputs and outputs, strong and weak decay, and the 32K-token GDN
in-projection shape fed straight from the fused GEMM's output columns.

Tolerance (float32 arithmetic, unit roundoff 2^-24): per (token, head),
||o - o_ref|| <= tau * ||S_ref,t||_F * ||q_t|| with tau = 2e-4, and the final
state ||S - S_ref||_F <= tau * ||S_ref||_F.  Within a chunk every quantity is
a sum of <= 64 + 128 + 128 products of magnitude <= ||S|| ||q|| (keys and
queries normalized, decay ratios <= 1, 0 <= beta <= 1); the state update is a
contraction (||exp(g)(I - beta k k^T)||_2 <= 1), so rounding errors of
earlier chunks do not grow, and over n chunks they add like sqrt(n) for
independent roundings; 2e-4 covers 512 chunks of ~1e-5 with a margin."""
import numpy as np
import pytest
import torch

import bit_linear_layer_amd as nv
import workloads as W
from oracle import nvfp4_oracle as O
from tests.gpu_util import DEV, say

pytestmark = pytest.mark.gpu
TAU = 2e-4


def inputs(rng, T, hk, hv, decay_scale=1.0):
    q = rng.standard_normal((T, hk, 128))
    k = rng.standard_normal((T, hk, 128))
    v = rng.standard_normal((T, hv, 128))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, hv)) * 2))
    a_log = np.log(rng.uniform(1, 16, hv))
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), hv))
    dt_bias = dt + np.log(-np.expm1(-dt))
    g = -np.exp(a_log) * np.log1p(np.exp(rng.standard_normal((T, hv)) + dt_bias)) * decay_scale
    return q, k, v, beta, g


def to_dev(x, dtype, T):
    a = torch.from_numpy(np.ascontiguousarray(x.reshape(T, -1), dtype=np.float32))
    return a.to(dtype).to(DEV)


def check(o_gpu, s_gpu, q, k, v, beta, g, normalize=True, s0=None, out_bf16=False):
    o_ref, s_ref = O.gdn_recurrence(q, k, v, beta, g, s0=s0, normalize=normalize)
    T, hv = o_ref.shape[0], o_ref.shape[1]
    qq = O.l2_normalize(q) / np.sqrt(128) if normalize else q
    rep = hv // q.shape[1]
    qn = np.linalg.norm(np.repeat(qq, rep, axis=1), axis=-1)  # [T, Hv]
    # ||S_ref,t||_F along the sequence, from a second oracle pass in pieces
    snorm = np.empty((T, hv))
    s = None if s0 is None else np.array(s0, dtype=np.float64)
    for t0 in range(0, T, 64):
        sl = slice(t0, min(T, t0 + 64))
        _, s_chunk = O.gdn_recurrence(q[sl], k[sl], v[sl], beta[sl], g[sl], s0=s, normalize=normalize)
        snorm[sl] = np.linalg.norm(s_chunk.reshape(hv, -1), axis=1)[None, :]  # chunk-end norm as the chunk's scale
        s = s_chunk
    og = o_gpu.float().cpu().numpy().reshape(T, hv, 128).astype(np.float64)
    err = np.linalg.norm(og - o_ref, axis=-1)
    bound = TAU * np.maximum(snorm, np.linalg.norm(s_ref.reshape(hv, -1), axis=1)[None, :]) * qn + 1e-30
    if out_bf16:  # rounding the output to bf16 adds at most half an ulp per element
        bound = bound + 2.0 ** -8 * np.linalg.norm(o_ref, axis=-1)
    worst = float(np.max(err / bound))
    assert worst <= 1.0, f"output error {worst:.3g} x the bound"
    if s_gpu is not None:
        sg = s_gpu.cpu().numpy().astype(np.float64)
        e = np.linalg.norm((sg - s_ref).reshape(hv, -1), axis=1) / np.linalg.norm(s_ref.reshape(hv, -1), axis=1)
        assert e.max() <= TAU, f"final state error {e.max():.3g}"
    return worst


@pytest.mark.parametrize("T,hk,hv", [(1, 1, 1), (63, 1, 2), (64, 2, 2), (130, 1, 8), (200, 2, 6), (1000, 1, 3)])
def test_gdn_matches_sequential_oracle(T, hk, hv):
    say(f"gdn {T}x{hk}/{hv}")
    rng = np.random.default_rng(T + hv)
    q, k, v, beta, g = inputs(rng, T, hk, hv)
    o, s = nv.gdn_recurrence(to_dev(q, torch.float32, T), to_dev(k, torch.float32, T), to_dev(v, torch.float32, T),
                             to_dev(beta, torch.float32, T), to_dev(g, torch.float32, T), hk, hv, return_state=True)
    torch.cuda.synchronize()
    check(o, s, q.astype(np.float32), k.astype(np.float32), v.astype(np.float32), beta.astype(np.float32),
          g.astype(np.float32))


@pytest.mark.parametrize("decay_scale", [0.0, 0.01, 30.0])
def test_gdn_decay_regimes_and_initial_state(decay_scale):
    """No decay (pure delta rule), weak decay, and decay strong enough that
    a chunk forgets its start (exp(gamma) underflows inside the chunk)."""
    say(f"gdn decay x{decay_scale}")
    rng = np.random.default_rng(11)
    T, hk, hv = 300, 1, 2
    q, k, v, beta, g = inputs(rng, T, hk, hv, decay_scale)
    s0 = rng.standard_normal((hv, 128, 128)) * 0.1
    f = lambda x: to_dev(x, torch.float32, T)
    o, s = nv.gdn_recurrence(f(q), f(k), f(v), f(beta), f(g), hk, hv,
                             s0=torch.from_numpy(s0.astype(np.float32)).to(DEV), return_state=True)
    torch.cuda.synchronize()
    check(o, s, *(x.astype(np.float32) for x in (q, k, v, beta, g)), s0=s0.astype(np.float32))


def test_gdn_raw_qk_bf16_in_bf16_out():
    """Unnormalized (pre-normalized by the caller) q/k, bf16 inputs and output."""
    say("gdn bf16")
    rng = np.random.default_rng(12)
    T, hk, hv = 257, 2, 4
    q, k, v, beta, g = inputs(rng, T, hk, hv)
    q = O.l2_normalize(q) / np.sqrt(128)
    k = O.l2_normalize(k)
    qb, kb, vb, bb, gb = (to_dev(x, torch.bfloat16, T) for x in (q, k, v, beta, g))
    o = nv.gdn_recurrence(qb, kb, vb, bb, gb, hk, hv, normalize_qk=False, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    back = lambda t, shape: W.bf16_to_f32_numpy(t).reshape(shape)
    check(o, None, back(qb, q.shape), back(kb, k.shape), back(vb, v.shape), back(bb, beta.shape),
          back(gb, g.shape), normalize=False, out_bf16=True)


def test_gdn_from_fused_in_projection_columns():
    """The 32K-token GDN in-projection: q/k/v/b/a columns of the fused GEMM's
    float32 output (gates in the epilogue) feed the recurrence directly;
    checked against the oracle on 2 of the 48 value heads, full length."""
    say("gdn 32768 from in-proj")
    wl = W.gdn_in_proj()
    x = wl.x.to(DEV)
    from tests.gpu_util import weight_segments
    wq, offs, sg = weight_segments([(n, t.to(DEV)) for n, t in wl.weights])
    a = nv.quantize(x)
    gate = dict(b_segment=4, a_segment=5, A_log=wl.extra["A_log"].to(DEV), dt_bias=wl.extra["dt_bias"].to(DEV))
    out = nv.gemm_fused_segments(a, wq, offs, sg, gate, out_dtype=torch.float32)
    del a, x
    q, k, v = out[:, offs[0]:offs[1]], out[:, offs[1]:offs[2]], out[:, offs[2]:offs[3]]
    beta, g = out[:, offs[4]:offs[5]], out[:, offs[5]:offs[6]]
    hk, hv = (offs[1] - offs[0]) // 128, (offs[3] - offs[2]) // 128
    o = nv.gdn_recurrence(q, k, v, beta, g, hk, hv)
    torch.cuda.synchronize()
    T = out.shape[0]
    for h in (0, 47):
        kh = h // (hv // hk)
        qs = q[:, kh * 128:(kh + 1) * 128].cpu().numpy().reshape(T, 1, 128)
        ks = k[:, kh * 128:(kh + 1) * 128].cpu().numpy().reshape(T, 1, 128)
        vs = v[:, h * 128:(h + 1) * 128].cpu().numpy().reshape(T, 1, 128)
        bs = beta[:, h:h + 1].cpu().numpy()
        gs = g[:, h:h + 1].cpu().numpy()
        check(o[:, h * 128:(h + 1) * 128], None, qs, ks, vs, bs, gs)
