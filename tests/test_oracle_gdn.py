"""Pins of the oracle's gated delta-rule recurrence against closed forms
(pure decay, exact key-value storage, overwrite along a repeated key, the
partial write), an exact-fraction evaluation, contraction, head sharing and
normalization invariance.  Two plausible mistakes (a flipped erase sign,
an erase term without the decay) fail the partial-write pin."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import nvfp4_oracle as O


def rnd(rng, *shape):
    return rng.standard_normal(shape)


def test_zero_write_strength_is_pure_decay():
    rng = np.random.default_rng(0)
    T, hk, hv, d = 7, 1, 2, 5
    q, k, v = rnd(rng, T, hk, d), rnd(rng, T, hk, d), rnd(rng, T, hv, d)
    g = -np.abs(rnd(rng, T, hv)) * 0.3
    s0 = rnd(rng, hv, d, d)
    o, s = O.gdn_recurrence(q, k, v, np.zeros((T, hv)), g, s0=s0, normalize=False)
    gam = np.exp(np.cumsum(g, axis=0))  # [T, Hv]
    for t in range(T):
        for h in range(hv):
            assert np.allclose(o[t, h], gam[t, h] * s0[h] @ q[t, 0], rtol=1e-12, atol=1e-12)
    assert np.allclose(s, gam[-1][:, None, None] * s0, rtol=1e-12)


def test_orthonormal_keys_store_values_exactly():
    rng = np.random.default_rng(1)
    d = 6
    basis = np.linalg.qr(rnd(rng, d, d))[0]  # orthonormal columns
    k = basis.T[:, None, :]                   # T = d tokens, key t = basis vector t
    v = rnd(rng, d, 1, d)
    o, s = O.gdn_recurrence(k, k, v, np.ones((d, 1)), np.zeros((d, 1)), normalize=False)
    for j in range(d):
        assert np.allclose(s[0] @ basis[:, j], v[j, 0], atol=1e-12)
    # reading with the last key returns the last value
    assert np.allclose(o[-1, 0], v[-1, 0], atol=1e-12)


def test_repeated_key_overwrites_and_leaves_orthogonal_directions():
    rng = np.random.default_rng(2)
    d = 4
    kk = np.array([1.0, 0, 0, 0])
    other = np.array([0, 1.0, 0, 0])
    k = np.stack([other, kk, kk])[:, None, :]
    v = rnd(rng, 3, 1, d)
    _, s = O.gdn_recurrence(k, k, v, np.ones((3, 1)), np.zeros((3, 1)), normalize=False)
    assert np.allclose(s[0] @ kk, v[2, 0], atol=1e-12)     # the second write replaced the first
    assert np.allclose(s[0] @ other, v[0, 0], atol=1e-12)  # an orthogonal association survives


def test_partial_write_closed_form():
    rng = np.random.default_rng(3)
    d = 5
    kk = O.l2_normalize(rnd(rng, d))
    perp = O.l2_normalize(rnd(rng, d) - (rnd(rng, d) @ kk) * kk)
    perp = O.l2_normalize(perp - (perp @ kk) * kk)
    s0 = rnd(rng, 1, d, d)
    v = rnd(rng, 1, 1, d)
    b, gg = 0.37, -0.2
    _, s = O.gdn_recurrence(kk[None, None], kk[None, None], v, np.array([[b]]), np.array([[gg]]), s0=s0,
                            normalize=False)
    a = np.exp(gg)
    assert np.allclose(s[0] @ kk, (1 - b) * a * s0[0] @ kk + b * v[0, 0], atol=1e-12)
    assert np.allclose(s[0] @ perp, a * s0[0] @ perp, atol=1e-12)


def test_exact_fraction_recurrence():
    """alpha = 1 (g = 0), rational beta and data: the float64 oracle agrees
    with S <- S (I - beta k k^T) + beta v k^T evaluated in exact fractions."""
    T, d = 4, 3
    rng = np.random.default_rng(4)
    k = rng.integers(-3, 4, size=(T, 1, d)).astype(np.float64) / 4
    q = rng.integers(-3, 4, size=(T, 1, d)).astype(np.float64) / 4
    v = rng.integers(-5, 6, size=(T, 1, d)).astype(np.float64) / 2
    beta = np.array([[0.25], [0.5], [0.75], [1.0]])
    o, s = O.gdn_recurrence(q, k, v, beta, np.zeros((T, 1)), normalize=False)
    S = [[Fraction(0)] * d for _ in range(d)]
    for t in range(T):
        kt = [Fraction(x) for x in k[t, 0]]
        vt = [Fraction(x) for x in v[t, 0]]
        b = Fraction(beta[t, 0])
        sk = [sum(S[i][j] * kt[j] for j in range(d)) for i in range(d)]
        S = [[S[i][j] - b * sk[i] * kt[j] + b * vt[i] * kt[j] for j in range(d)] for i in range(d)]
        ot = [sum(S[i][j] * Fraction(q[t, 0, j]) for j in range(d)) for i in range(d)]
        assert np.allclose(o[t, 0], [float(x) for x in ot], rtol=1e-13, atol=1e-13)
    assert np.allclose(s[0], [[float(x) for x in row] for row in S], rtol=1e-13, atol=1e-13)


def test_state_norm_contracts_without_writes_of_new_values():
    rng = np.random.default_rng(5)
    T, d = 50, 8
    k = rnd(rng, T, 1, d)
    beta = 1 / (1 + np.exp(-rnd(rng, T, 1)))
    g = -np.abs(rnd(rng, T, 1)) * 0.05
    s0 = rnd(rng, 1, d, d)
    norms = [np.linalg.norm(s0)]
    s = s0
    for t in range(T):
        _, s = O.gdn_recurrence(k[t:t + 1], k[t:t + 1], np.zeros((1, 1, d)), beta[t:t + 1], g[t:t + 1], s0=s)
        norms.append(np.linalg.norm(s))
    assert all(b <= a * (1 + 1e-12) for a, b in zip(norms, norms[1:]))


def test_value_heads_share_key_heads():
    rng = np.random.default_rng(6)
    T, d = 6, 4
    q, k, v = rnd(rng, T, 1, d), rnd(rng, T, 1, d), rnd(rng, T, 3, d)
    beta, g = 1 / (1 + np.exp(-rnd(rng, T, 3))), -np.abs(rnd(rng, T, 3)) * 0.1
    o, s = O.gdn_recurrence(q, k, v, beta, g)
    for h in range(3):
        oh, sh = O.gdn_recurrence(q, k, v[:, h:h + 1], beta[:, h:h + 1], g[:, h:h + 1])
        assert np.allclose(o[:, h], oh[:, 0], rtol=1e-13) and np.allclose(s[h], sh[0], rtol=1e-13)


def test_normalization_makes_q_and_k_scale_free():
    rng = np.random.default_rng(7)
    T, d = 5, 6
    q, k, v = rnd(rng, T, 1, d), rnd(rng, T, 1, d), rnd(rng, T, 2, d)
    beta, g = np.full((T, 2), 0.6), np.full((T, 2), -0.05)
    o1, _ = O.gdn_recurrence(q, k, v, beta, g)
    o2, _ = O.gdn_recurrence(q * 3.7, k * 0.01, v, beta, g)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-13)


def flipped_sign(s, k, v, b, a):
    return a * s + a * b * np.outer(s @ k, k) + b * np.outer(v, k)


def erase_without_decay(s, k, v, b, a):
    return a * s - b * np.outer(s @ k, k) + b * np.outer(v, k)


@pytest.mark.parametrize("mistake", [flipped_sign, erase_without_decay])
def test_planted_mistakes_fail_the_partial_write_pin(mistake):
    rng = np.random.default_rng(8)
    d = 5
    kk = O.l2_normalize(rnd(rng, d))
    s0, v = rnd(rng, d, d), rnd(rng, d)
    b, a = 0.37, np.exp(-0.2)
    s = mistake(s0, kk, v, b, a)
    assert not np.allclose(s @ kk, (1 - b) * a * s0 @ kk + b * v, atol=1e-9)


def test_normalized_query_reads_stored_value_scaled_by_inverse_sqrt_dk():
    """Closed form of the normalized read.  Orthonormal keys written with
    beta = 1 and no decay store v exactly along each key; a query c * k_j
    with any c != 0 normalizes to sign(c) k_j and is scaled by dk^-1/2, so
    the read is sign(c) v_j / sqrt(dk) at the head width of the GPU path
    (128), and a query along a key not yet written reads zero.  Dropping the
    query scale, normalizing over another axis, or leaving q unnormalized
    all fail."""
    rng = np.random.default_rng(9)
    d, n, hk, hv = 128, 5, 2, 4
    rep = hv // hk
    basis = np.linalg.qr(rnd(rng, d, d))[0].T           # rows: orthonormal keys
    key = lambda kh, j: basis[n * kh + j]               # slot j of key head kh
    T = 2 * n
    k, q = np.zeros((T, hk, d)), np.zeros((T, hk, d))
    v = rnd(rng, T, hv, d)
    beta = np.zeros((T, hv))
    coef = np.zeros((T, hk))
    slot = np.zeros((T, hk), dtype=int)
    for t in range(T):
        for kh in range(hk):
            if t < n:   # token t writes slot t of every key head, key scaled arbitrarily
                k[t, kh] = key(kh, t) * (0.01 + 3.0 * t)
                beta[t, kh * rep:(kh + 1) * rep] = 1.0
            else:       # no writes (beta = 0) along a spare key
                k[t, kh] = basis[2 * n + kh]
            slot[t, kh] = (t + 3 * kh) % n
            coef[t, kh] = (-1) ** (t + kh) * (0.2 + 7.0 * rng.random())
            q[t, kh] = coef[t, kh] * key(kh, slot[t, kh])
    o, _ = O.gdn_recurrence(q, k, v, beta, np.zeros((T, hv)), normalize=True)
    checked = 0
    for t in range(T):
        for h in range(hv):
            kh = h // rep
            j = slot[t, kh]
            expect = np.sign(coef[t, kh]) * v[j, h] / np.sqrt(128.0) if j <= t else np.zeros(d)
            assert np.allclose(o[t, h], expect, rtol=1e-10, atol=1e-12)
            checked += j > t
    assert checked > 0   # some queries read slots not yet written


def test_query_scale_alone_leaves_normalized_output_unchanged():
    """Scaling q alone (k fixed) by any positive factor changes nothing with
    normalize=True; without normalization the output scales with q."""
    rng = np.random.default_rng(10)
    T, d = 6, 16
    q, k, v = rnd(rng, T, 1, d), rnd(rng, T, 1, d), rnd(rng, T, 2, d)
    beta, g = np.full((T, 2), 0.7), np.full((T, 2), -0.1)
    o1, _ = O.gdn_recurrence(q, k, v, beta, g)
    o2, _ = O.gdn_recurrence(q * 41.0, k, v, beta, g)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-14)
    o3, _ = O.gdn_recurrence(q, k, v, beta, g, normalize=False)
    o4, _ = O.gdn_recurrence(q * 41.0, k, v, beta, g, normalize=False)
    assert np.allclose(o4, 41.0 * o3, rtol=1e-12)
