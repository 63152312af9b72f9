"""Pins of the oracle's exact-or-approximate (piecewise) tail.

Checked against dense softmax attention, written out here from its definition, in the cases
where the expansion is exact or its error order is known: every block routed; key blocks
without spread (the zero-order term is then exact for any routing); value rows all equal to
one (the output must be exactly one, which pins the token counts in the denominator); and
blocks sharing one first-order matrix, where the error must fall as the square of the
spread (a dropped or mis-signed first-order term leaves a linear error).
"""
import math

import numpy as np
import pytest

from oracle import pisa

RNG = np.random.default_rng(77)
B = 64


def dense_attention(q, k, v):
    """softmax(q k^T / sqrt(d)) v, row by row."""
    z = q @ k.T / math.sqrt(q.shape[1])
    z -= z.max(axis=1, keepdims=True)
    w = np.exp(z)
    return (w / w.sum(axis=1, keepdims=True)) @ v


def run(q, k, v, top_k, proj=None):
    d = q.shape[1]
    p = RNG.standard_normal((d, d)) if proj is None else proj
    out, r = pisa.forward_head(q, k, v, p, p, B, top_k)
    return out, r


def test_every_block_routed_is_dense_attention():
    d, nq, nkv = 16, 2 * B, 5 * B + 9
    q, k, v = (RNG.standard_normal((n, d)) for n in (nq, nkv, nkv))
    out, _ = run(q, k, v, top_k=6)
    assert np.allclose(out, dense_attention(q, k, v), rtol=0, atol=1e-12)


@pytest.mark.parametrize("top_k", [0, 1, 3])
def test_constant_key_blocks_are_exact(top_k):
    """Keys constant inside each block: exp(q.k) is exactly a_j on the whole block, H_j = 0,
    so the piecewise output equals dense attention whatever is routed (also a partial
    last block)."""
    d, nq, nkv = 16, 2 * B, 4 * B + 20
    nb = -(-nkv // B)
    centers = 1.5 * RNG.standard_normal((nb, d))
    k = np.repeat(centers, B, axis=0)[:nkv]
    q = RNG.standard_normal((nq, d))
    v = RNG.standard_normal((nkv, d))
    out, _ = run(q, k, v, top_k)
    assert np.allclose(out, dense_attention(q, k, v), rtol=0, atol=1e-12)


@pytest.mark.parametrize("top_k", [0, 2])
def test_unit_values_give_unit_output(top_k):
    """v = 1 everywhere: H_j = 0 and each block's numerator equals its denominator term
    (a_j Vsum_j = a_j n_j), so o = 1 exactly for any keys, including a partial block."""
    d, nq, nkv = 16, B + 30, 4 * B + 10
    q = RNG.standard_normal((nq, d))
    k = 2.0 * RNG.standard_normal((nkv, d))
    v = np.ones((nkv, d))
    out, _ = run(q, k, v, top_k)
    assert np.allclose(out, 1.0, rtol=0, atol=1e-12)


def shared_first_order(eps, d=16, nb=6, nq=B):
    """Blocks k = c_j + eps delta_n (sum_n delta_n = 0) and v = b_j + w_n with the same
    delta and w in every block: H_j = eps sum_n delta_n^T w_n is the same matrix for all j,
    so H_bar is exact and only second-order terms remain."""
    rng = np.random.default_rng(5)
    delta = rng.standard_normal((B, d))
    delta -= delta.mean(axis=0)
    w = rng.standard_normal((B, d))
    c = rng.standard_normal((nb, d))
    bvec = rng.standard_normal((nb, d))
    k = (c[:, None, :] + eps * delta[None]).reshape(nb * B, d)
    v = (bvec[:, None, :] + w[None]).reshape(nb * B, d)
    q = 1.5 * rng.standard_normal((nq, d))
    proj = rng.standard_normal((d, d))
    return q, k, v, proj


def test_shared_first_order_error_is_second_order():
    errs = []
    for eps in (4e-2, 2e-2, 1e-2):
        q, k, v, proj = shared_first_order(eps)
        out, _ = pisa.forward_head(q, k, v, proj, proj, B, 2)
        errs.append(np.abs(out - dense_attention(q, k, v)).max())
    r1, r2 = errs[0] / errs[1], errs[1] / errs[2]
    assert 3.5 < r1 < 4.5 and 3.5 < r2 < 4.5, errs
    assert errs[2] < 1e-3


def test_first_order_term_matters():
    """Same blocks: without the first-order term the error would be linear in the spread;
    the piecewise output is much closer to dense attention than the zero-order-only sum
    (computed here from the definitions with H_bar = 0)."""
    q, k, v, proj = shared_first_order(1e-2)
    out, r = pisa.forward_head(q, k, v, proj, proj, B, 2)
    k_bar, vsum, counts, H = pisa.block_stats(k, v, B)
    zero = np.concatenate([pisa.tail_rows(q[i * B:(i + 1) * B], k, v, r.idx[i], k_bar, vsum,
                                          counts, np.zeros_like(H[0]), B)
                           for i in range(q.shape[0] // B)])
    dense = dense_attention(q, k, v)
    assert np.abs(out - dense).max() * 20 < np.abs(zero - dense).max()


def test_block_stats_definitions():
    """Centroid, value sums, counts and H_j on a two-token partial block by hand."""
    d = 3
    k = np.zeros((B + 2, d))
    v = np.zeros((B + 2, d))
    k[B], k[B + 1] = [1.0, 2.0, 3.0], [3.0, 2.0, 1.0]
    v[B], v[B + 1] = [1.0, 0.0, 0.0], [0.0, 1.0, 0.0]
    k_bar, vsum, counts, H = pisa.block_stats(k, v, B)
    assert np.array_equal(counts, [B, 2])
    assert np.allclose(k_bar[1], [2.0, 2.0, 2.0])
    assert np.allclose(vsum[1], [1.0, 1.0, 0.0])
    # deviations (-1, 0, 1) and (1, 0, -1): H = dev1^T v1 + dev2^T v2
    want = np.array([[-1.0, 1.0, 0.0], [0.0, 0.0, 0.0], [1.0, -1.0, 0.0]])
    assert np.allclose(H[1], want)
