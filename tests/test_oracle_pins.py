"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test is chosen so that a plausible mistake in the oracle (a dropped term, a wrong
sign, scale or index, a transposed operand, a wrong tie rule, pooling over padding) fails
at least one of them. None of them re-calls the oracle's own formula for its expected
value: expected values come from brute-force token loops (tests/_brute.py), from library
routines (torch scaled_dot_product_attention in float64), from closed forms, or from
invariants.
"""
import itertools
import math

import numpy as np
import pytest

from oracle import sla_oracle as so
from tests import _brute as bf

RNG = np.random.default_rng(1234)


def rand_head(nq, nk, d, rng=RNG, scale=1.0):
    q = rng.standard_normal((nq, d)) * scale
    k = rng.standard_normal((nk, d)) * scale
    v = rng.standard_normal((nk, d))
    pq = rng.standard_normal((d, d)) / math.sqrt(d)
    pk = rng.standard_normal((d, d)) / math.sqrt(d)
    al = rng.uniform(0, 1, d)
    return q, k, v, pq, pk, al


# --------------------------------------------------------------------------- special cases
@pytest.mark.parametrize("nq,nk,d", [(256, 256, 16), (200, 330, 32), (64, 640, 16)])
def test_all_blocks_alpha1_is_dense_softmax_attention(nq, nk, d):
    """top_k = all blocks and alpha = 1 reduce to dense softmax attention (library routine)."""
    torch = pytest.importorskip("torch")
    q, k, v, pq, pk, _ = rand_head(nq, nk, d)
    nbk = so.n_blocks(nk, 32)
    r = so.forward_head(q, k, v, pq, pk, np.ones(d), 32, nbk)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None]).numpy()[0]
    assert np.abs(r.out - ref).max() <= 1e-12 * np.abs(ref).max()


@pytest.mark.parametrize("nq,nk,d,b", [(96, 160, 8, 32), (64, 100, 12, 16)])
def test_topk0_alpha0_is_linear_attention(nq, nk, d, b):
    """top_k = 0 and alpha = 0 reduce to ReLU linear attention over every key (brute force)."""
    q, k, v, pq, pk, _ = rand_head(nq, nk, d)
    r = so.forward_head(q, k, v, pq, pk, np.zeros(d), b, 0)
    for n in range(0, nq, 7):
        ref = bf.linear_attention_row(q[n].tolist(), k.tolist(), v.tolist())
        assert np.allclose(r.out[n], ref, rtol=1e-11, atol=1e-12)


def test_mix_endpoints_and_affinity():
    q, k, v, pq, pk, al = rand_head(128, 192, 16)
    r1 = so.forward_head(q, k, v, pq, pk, np.ones(16), 32, 2)
    r0 = so.forward_head(q, k, v, pq, pk, np.zeros(16), 32, 2)
    ra = so.forward_head(q, k, v, pq, pk, al, 32, 2)
    assert np.array_equal(r1.out, r1.o_s)
    assert np.array_equal(r0.out, r0.o_l)
    # affine in alpha, channel by channel
    assert np.allclose(ra.out, al * r1.out + (1 - al) * r0.out, rtol=1e-13, atol=1e-14)
    # the two branches do not depend on alpha
    assert np.array_equal(ra.o_s, r1.o_s) and np.array_equal(ra.o_l, r0.o_l)


# --------------------------------------------------------------------------- brute force
@pytest.mark.parametrize("nq,nk,d,b,k", [(96, 96, 8, 16, 2), (70, 150, 8, 16, 3), (48, 160, 4, 32, 1)])
def test_branches_match_token_brute_force(nq, nk, d, b, k):
    """Sparse branch = softmax over the routed tokens; linear branch = ReLU linear attention
    over exactly the tokens NOT routed (partial last blocks included)."""
    q, kk, v, pq, pk, al = rand_head(nq, nk, d)
    r = so.forward_head(q, kk, v, pq, pk, al, b, k)
    # routing by brute force: pooled means, projections and scores by loops
    nbq, nbk = so.n_blocks(nq, b), so.n_blocks(nk, b)
    qt = [[bf.dot(bf.pooled_mean(q.tolist(), i, b), pq[:, c].tolist()) for c in range(d)] for i in range(nbq)]
    kt = [[bf.dot(bf.pooled_mean(kk.tolist(), j, b), pk[:, c].tolist()) for c in range(d)] for j in range(nbk)]
    for i in range(nbq):
        s = [bf.dot(qt[i], kt[j]) for j in range(nbk)]
        # best k-subset by enumeration (scores are distinct for random inputs)
        best = max(itertools.combinations(range(nbk), k), key=lambda c: sum(s[j] for j in c))
        assert list(r.route.idx[i]) == sorted(best)
        sel = set(best)
        toks_s = [t for j in sorted(sel) for t in bf.block_tokens(j, nk, b)]
        toks_l = [t for j in range(nbk) if j not in sel for t in bf.block_tokens(j, nk, b)]
        for n in bf.block_tokens(i, nq, b)[::5]:
            os_ = bf.softmax_attention_row(q[n].tolist(), [kk[t].tolist() for t in toks_s],
                                           [v[t].tolist() for t in toks_s])
            ol = bf.linear_attention_row(q[n].tolist(), [kk[t].tolist() for t in toks_l],
                                         [v[t].tolist() for t in toks_l])
            assert np.allclose(r.o_s[n], os_, rtol=1e-11, atol=1e-13)
            assert np.allclose(r.o_l[n], ol, rtol=1e-10, atol=1e-13)
            want = [a * x + (1 - a) * y for a, x, y in zip(al, os_, ol)]
            assert np.allclose(r.out[n], want, rtol=1e-10, atol=1e-13)


def test_pool_over_valid_tokens_only():
    """The partial last block is averaged over its valid tokens, not over the block size."""
    x = RNG.standard_normal((3 * 64 + 16, 8))
    pooled = so.pool_blocks(x, 64)
    assert pooled.shape == (4, 8)
    for j in range(4):
        assert np.allclose(pooled[j], bf.pooled_mean(x.tolist(), j, 64), rtol=1e-14, atol=1e-15)
    # a value in the padded region of a larger buffer cannot reach the result
    assert np.allclose(pooled[3], x[192:].sum(axis=0) / 16, rtol=1e-14)


def test_sparse_rows_are_normalised():
    """Softmax rows sum to one: with V = 1 the sparse branch returns exactly 1."""
    q, k, v, pq, pk, _ = rand_head(128, 256, 16)
    r = so.forward_head(q, k, np.ones_like(v), pq, pk, np.ones(16), 32, 3)
    assert np.allclose(r.out, 1.0, rtol=0, atol=1e-14)


def test_empty_complement_and_empty_selection():
    q, k, v, pq, pk, al = rand_head(64, 128, 8)
    full = so.forward_head(q, k, v, pq, pk, al, 32, 4)        # all 4 blocks selected
    assert np.array_equal(full.o_l, np.zeros_like(full.o_l))
    none = so.forward_head(q, k, v, pq, pk, al, 32, 0)        # nothing selected
    assert np.array_equal(none.o_s, np.zeros_like(none.o_s))
    assert none.route.idx.shape == (2, 0)


# --------------------------------------------------------------------------- router
def test_router_closed_form_and_ties():
    """proj = I and constant blocks give closed-form scores s_ij = a_i . b_j; duplicated key
    blocks tie exactly and the lower index wins."""
    d, b = 4, 8
    nbq, nbk = 3, 6
    a = np.array([[1, 0, 0, 0], [0, 1, 0, 0], [1, 1, 0, 0]], float)
    bb = np.array([[5, 0, 0, 0], [1, 9, 0, 0], [5, 0, 0, 0], [2, 2, 0, 0], [0, 0, 7, 0], [1, 9, 0, 0]], float)
    q = np.repeat(a, b, axis=0)
    k = np.repeat(bb, b, axis=0)
    eye = np.eye(d)
    r = so.route_head(q, k, eye, eye, b, 2)
    assert np.array_equal(r.scores, a @ bb.T)
    # row 0 scores [5,1,5,2,0,1]: blocks 0 and 2 tie at 5 -> both kept (k=2)
    assert r.idx[0].tolist() == [0, 2]
    # row 1 scores [0,9,0,2,0,9]: 1 and 5 tie at 9 -> both kept
    assert r.idx[1].tolist() == [1, 5]
    # row 2 scores [5,10,5,4,0,10]: 1 and 5 -> kept
    assert r.idx[2].tolist() == [1, 5]
    r1 = so.route_head(q, k, eye, eye, b, 1)
    assert r1.idx[:, 0].tolist() == [0, 1, 1]          # ties go to the lower index
    r3 = so.route_head(q, k, eye, eye, b, 3)
    assert r3.idx[0].tolist() == [0, 2, 3]
    assert r3.idx[1].tolist() == [1, 3, 5]             # 9, 9, then 2
    assert r3.idx[2].tolist() == [0, 1, 5]             # 10, 10, then 5 (block 0 beats block 2)


def test_projection_orientation():
    """x @ P with P stored [d_in, d_out]: a non-symmetric P that routes channel 0 of the
    pooled query onto output channel 1 must change the selection accordingly."""
    d, b = 2, 4
    q = np.repeat(np.array([[1.0, 0.0]]), b, axis=0)
    k = np.repeat(np.array([[1.0, 0.0], [0.0, 1.0]]), b, axis=0)
    P = np.array([[0.0, 1.0], [0.0, 0.0]])   # (1,0) @ P = (0,1)
    r = so.route_head(q, k, P, np.eye(d), b, 1)
    assert r.idx[0].tolist() == [1]
    r = so.route_head(q, k, P.T, np.eye(d), b, 1)   # (1,0) @ P^T = (0,0): all tie -> lowest
    assert r.idx[0].tolist() == [0]


# --------------------------------------------------------------------------- invariances
def test_permutation_within_blocks():
    q, k, v, pq, pk, al = rand_head(128, 192, 16)
    b = 32
    base = so.forward_head(q, k, v, pq, pk, al, b, 2)
    # permute keys (same permutation on K and V) inside every key block
    perm = np.concatenate([j * b + RNG.permutation(min(b, 192 - j * b)) for j in range(6)])
    pr = so.forward_head(q, k[perm], v[perm], pq, pk, al, b, 2)
    assert np.array_equal(pr.route.idx, base.route.idx)
    assert np.allclose(pr.out, base.out, rtol=1e-12, atol=1e-14)
    # permute query rows inside every query block: outputs permute the same way
    qp = np.concatenate([i * b + RNG.permutation(b) for i in range(4)])
    pr = so.forward_head(q[qp], k, v, pq, pk, al, b, 2)
    assert np.array_equal(pr.route.idx, base.route.idx)
    assert np.allclose(pr.out, base.out[qp], rtol=1e-12, atol=1e-14)


def test_complement_equals_total_minus_selected():
    """SPLA page, section 2.2: the linear term over the unselected blocks equals the global
    linear term minus the term over the selected blocks (here in summary space)."""
    q, k, v, pq, pk, al = rand_head(96, 320, 8)
    b, top = 32, 4
    r = so.forward_head(q, k, v, pq, pk, al, b, top)
    S, z = so.block_summaries(k, v, b)
    fq = np.maximum(q, 0)
    for i in range(3):
        sel = r.route.idx[i]
        Sc = S.sum(0) - S[sel].sum(0)
        zc = z.sum(0) - z[sel].sum(0)
        rows = slice(i * b, (i + 1) * b)
        ol = (fq[rows] @ Sc) / (fq[rows] @ zc + so.EPS)[:, None]
        assert np.allclose(ol, r.o_l[rows], rtol=1e-10, atol=1e-13)


def test_forward_wrapper_matches_head_function():
    from workloads import make_custom
    x = make_custom(2, 2, 100, 100, 8, 1, dtype="f32", block=32)
    out, idx = so.forward(x)
    for b in range(2):
        for h in range(2):
            r = so.forward_head(x.as_f64("q")[b, h], x.as_f64("k")[b, h], x.as_f64("v")[b, h],
                                x.proj_q.astype(float), x.proj_k.astype(float),
                                x.alpha[h].astype(float), 32, 1)
            assert np.array_equal(out[b, h], r.out)
            assert np.array_equal(idx[b, h], r.route.idx)
    rows = np.array([0, 5, 63, 64, 99])
    out2, _ = so.forward(x, heads=[(1, 0)], rows=rows)
    assert np.allclose(out2[1, 0, rows], out[1, 0, rows], rtol=1e-13, atol=1e-15)
    assert np.isnan(out2[0, 0]).all()
