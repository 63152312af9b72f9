"""Pins of the oracle's training-free (second-order Taylor) router.

The score is checked against what it approximates — the block's mean exponential attention
score computed token by token — on blocks whose covariance is diagonal by construction,
where the second-order expansion leaves only fourth-order terms; against closed forms
(zero variance, a two-value block); and for the properties a ranking score must have.
"""
import math

import numpy as np

from oracle import sla_oracle as so

RNG = np.random.default_rng(2024)


def exact_log_mass(q, keys):
    """log of the mean over the block's tokens of exp(tau q.k_t), token by token."""
    tau = 1.0 / math.sqrt(q.shape[0])
    z = tau * keys @ q
    m = z.max()
    return m + math.log(np.mean(np.exp(z - m)))


def diagonal_block(d, n, center, eps):
    """n tokens = center +- eps on one channel each (pairs), so that the sample mean is the
    centre and the sample covariance is exactly diagonal."""
    keys = np.repeat(center[None], n, axis=0)
    chans = RNG.integers(0, d, size=n // 2)
    for p, c in enumerate(chans):
        keys[2 * p, c] += eps
        keys[2 * p + 1, c] -= eps
    return keys


def test_zero_variance_block_is_scaled_dot_product():
    d = 16
    q = RNG.standard_normal((3, d))
    kb = RNG.standard_normal((5, d))
    s = so.taylor_scores(q, kb, np.zeros((5, d)))
    assert np.allclose(s, q @ kb.T / math.sqrt(d), rtol=0, atol=1e-15)


def test_two_value_block_variance_closed_form():
    """Tokens alternating between a and b: mean (a+b)/2, variance ((a-b)/2)^2 per channel;
    a partial block only counts its valid tokens."""
    d = 8
    a, b = RNG.standard_normal(d), RNG.standard_normal(d)
    x = np.stack([a if t % 2 == 0 else b for t in range(64 + 6)])
    v = so.block_variances(x, 64)
    assert np.allclose(v[0], ((a - b) / 2) ** 2, rtol=1e-13)
    assert np.allclose(v[1], ((a - b) / 2) ** 2, rtol=1e-13)      # 6 valid tokens, 3 + 3
    y = np.concatenate([x[:64], np.stack([a, a, b])])               # 3 valid: 2 a + 1 b
    w = so.block_variances(y, 64)
    assert np.allclose(w[1], (2.0 / 9.0) * (a - b) ** 2, rtol=1e-13)


def test_second_order_estimate_matches_token_mass():
    """On diagonal-covariance blocks the log score differs from the exact log mean
    exponential score only at fourth order in the spread."""
    d, n = 32, 64
    for eps, tol in ((1e-2, 1e-9), (3e-2, 1e-7)):
        for _ in range(5):
            q = RNG.standard_normal(d) * 2
            center = RNG.standard_normal(d)
            keys = diagonal_block(d, n, center, eps)
            s = so.taylor_scores(q[None], keys.mean(axis=0)[None],
                                 so.block_variances(keys, n))[0, 0]
            assert abs(s - exact_log_mass(q, keys)) < tol


def test_variance_raises_the_score_along_the_query():
    """Same mean: spread along channels the query weighs raises the score; spread where the
    query is zero does not change it."""
    d = 8
    q = np.zeros(d)
    q[:4] = RNG.standard_normal(4) + 2
    kb = np.tile(RNG.standard_normal(d), (3, 1))
    var = np.zeros((3, d))
    var[1, :4] = 0.5
    var[2, 4:] = 5.0
    s = so.taylor_scores(q[None], kb, var)[0]
    assert s[1] > s[0] and s[2] == s[0]


def test_route_reduces_to_dot_product_router_without_spread():
    """Constant key blocks (zero variance) and identity projections: the Taylor route picks
    exactly the blocks of the learnable router (tau > 0 does not change the order)."""
    d, b = 16, 64
    q = RNG.standard_normal((3 * b, d))
    kb = RNG.standard_normal((9, d))
    k = np.repeat(kb, b, axis=0)
    eye = np.eye(d)
    r1 = so.route_head(q, k, eye, eye, b, 4)
    r2 = so.route_head_taylor(q, k, b, 4)
    assert np.array_equal(r1.idx, r2.idx)
