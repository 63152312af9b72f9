"""Pins of the oracle's wrappers and bookkeeping: the near-tie flag that decides which GPU
selections may differ from the oracle's, the fp8 forward's composition (router, quantised
sparse branch, linear branch, mix), the literal-reading fp8 variant, and the all-heads
wrappers of the piecewise forward and of the router.

Expected values come from pure-Python token loops (tests/_brute.py), hand-built score rows
and closed-form error bounds; none re-calls the function under test to make its own
expected value.
"""
import math

import numpy as np
import pytest

from oracle import fp8
from oracle import pisa
from oracle import sla_oracle as so
from tests import _brute as bf
from workloads import Inputs, Problem, make_custom

RNG = np.random.default_rng(4321)


# --------------------------------------------------------------------------- near ties
def _flags(rows, k):
    s = np.array(rows, dtype=np.float64)
    g = so.boundary_gaps(s, k)
    return g, so.near_ties(s, g)


def test_boundary_gap_is_kth_minus_next_in_descending_order():
    g, f = _flags([[1.0, 5.0, 3.0, 4.0]], 2)
    assert g[0] == 1.0 and not f[0]            # 5 4 | 3 1
    g, f = _flags([[1.0, 5.0, 3.0, 4.0]], 1)
    assert g[0] == 1.0 and not f[0]            # 5 | 4 3 1
    g, f = _flags([[1.0, 5.0, 3.0, 4.0]], 3)
    assert g[0] == 2.0 and not f[0]            # 5 4 3 | 1


def test_exact_tie_at_the_boundary_is_flagged():
    g, f = _flags([[5.0, 3.0, 3.0, 1.0]], 2)
    assert g[0] == 0.0 and f[0]
    g, f = _flags([[5.0, 3.0, 3.0, 1.0]], 1)   # tie inside the kept set is harmless
    assert g[0] == 2.0 and not f[0]


def test_near_tie_threshold_is_relative_to_largest_magnitude():
    one = 1.0
    below = one - 0.9e-12
    above = one - 1.1e-12
    assert _flags([[one, below, 0.0]], 1)[1][0]
    assert not _flags([[one, above, 0.0]], 1)[1][0]
    # the scale is the row's largest |score|, here a negative entry outside the kept set
    g, f = _flags([[-4.0, one, one - 3e-12]], 1)
    assert math.isclose(g[0], 3e-12, rel_tol=1e-3) and f[0]
    g, f = _flags([[-2.0, one, one - 3e-12]], 1)
    assert not f[0]
    # scaling the whole row does not change the flag
    for sc in (1e-30, 1e30):
        assert _flags([[sc, sc * below, 0.0]], 1)[1][0]
        assert not _flags([[sc, sc * above, 0.0]], 1)[1][0]


@pytest.mark.parametrize("k", [0, 4])
def test_no_boundary_when_none_or_all_blocks_are_kept(k):
    g, f = _flags([[1.0, 1.0, 1.0, 1.0], [2.0, -1.0, 0.0, 3.0]], k)
    assert np.all(np.isinf(g)) and not f.any()


def test_gaps_match_a_python_sort_on_random_rows():
    s = RNG.standard_normal((20, 37))
    s[3, 5] = s[3, 9]                          # a planted tie
    for k in (1, 7, 36):
        g = so.boundary_gaps(s, k)
        for i in range(s.shape[0]):
            srt = sorted(s[i].tolist(), reverse=True)
            assert g[i] == srt[k - 1] - srt[k]


def test_route_flags_planted_ties_and_only_them():
    """Two identical key blocks that both outscore every other block for query block 0 tie
    at the top-1 boundary there, and the router flags exactly that row."""
    d, b = 8, 16
    q = RNG.standard_normal((4 * b, d))
    k = RNG.standard_normal((6 * b, d))
    k[1 * b:2 * b] += 10.0 * q[:b].mean(axis=0)  # block 1 aligned with query block 0
    k[4 * b:5 * b] = k[1 * b:2 * b]             # block 4 duplicates block 1
    eye = np.eye(d)
    r = so.route_head(q, k, eye, eye, b, 1)
    assert r.near_tie[0] and r.idx[0].tolist() == [1]
    for i in range(4):
        srt = sorted(r.scores[i].tolist(), reverse=True)
        assert bool(r.near_tie[i]) == (srt[0] == srt[1])


def test_check_masks_accepts_alternatives_only_on_flagged_rows():
    from tests.gpu_helpers import check_masks
    s = np.array([[5.0, 3.0, 3.0, 1.0], [5.0, 4.0, 3.0, 1.0]])
    g = so.boundary_gaps(s, 2)
    r = so.Route(so.select_topk(s, 2), s, g, so.near_ties(s, g))
    assert r.idx.tolist() == [[0, 1], [0, 1]]
    rows, near = check_masks(np.array([[[[0, 1], [0, 1]]]]), [[r]], 2)
    assert (rows, near) == (2, 0)
    rows, near = check_masks(np.array([[[[0, 2], [0, 1]]]]), [[r]], 2)   # the other tie
    assert (rows, near) == (2, 1)
    with pytest.raises(AssertionError):        # not a top-2 set of the tied row
        check_masks(np.array([[[[0, 3], [0, 1]]]]), [[r]], 2)
    with pytest.raises(AssertionError):        # an unflagged row must match exactly
        check_masks(np.array([[[[0, 1], [0, 2]]]]), [[r]], 2)
    with pytest.raises(AssertionError):        # not ascending
        check_masks(np.array([[[[2, 0], [0, 1]]]]), [[r]], 2)


# --------------------------------------------------------------------------- fp8 composition
def _brute_forward_fp8(x: Inputs):
    """The quantised forward of every (b, h) token by token: router from pooled means and
    projections, per-block power-of-two E4M3 quantisation of Q, K, V, the quantised sparse
    branch over the routed tiles, unquantised linear attention over the other key tokens,
    and the per-channel mix."""
    p = x.problem
    table = bf.e4m3_table()
    out = np.zeros((p.batch, p.heads, p.n_q, p.head_dim))
    nbq, nbk, blk = p.nbq, p.nbk, p.block

    def quant(rows):
        res, sc = [], []
        for j in range(-(-len(rows) // blk)):
            toks = bf.block_tokens(j, len(rows), blk)
            e = bf.pow2_block_exponent(max(abs(v) for t in toks for v in rows[t]))
            sc.append(2.0 ** e)
            res += [[bf.e4m3_nearest(v * 2.0 ** -e, table) for v in rows[t]] for t in toks]
        return res, sc

    for b in range(p.batch):
        for h in range(p.heads):
            q = x.as_f64("q")[b, h].tolist()
            k = x.as_f64("k")[b, h].tolist()
            v = x.as_f64("v")[b, h].tolist()
            pq = x.proj_q.astype(float).tolist()
            pk = x.proj_k.astype(float).tolist()
            d = len(q[0])

            def proj(vec, P):
                return [sum(vec[r] * P[r][c] for r in range(d)) for c in range(d)]
            qt = [proj(bf.pooled_mean(q, i, blk), pq) for i in range(nbq)]
            kt = [proj(bf.pooled_mean(k, j, blk), pk) for j in range(nbk)]
            q8, sq = quant(q)
            k8, sk = quant(k)
            v8, sv = quant(v)
            for i in range(nbq):
                s = [bf.dot(qt[i], kt[j]) for j in range(nbk)]
                sel = sorted(sorted(range(nbk), key=lambda j: (-s[j], j))[:p.top_k])
                tiles = [([k8[t] for t in bf.block_tokens(j, len(k), blk)], sk[j],
                          [v8[t] for t in bf.block_tokens(j, len(k), blk)], sv[j]) for j in sel]
                comp = [t for j in range(nbk) if j not in sel for t in bf.block_tokens(j, len(k), blk)]
                for n in bf.block_tokens(i, len(q), blk):
                    o_s = bf.fp8_attention_row(q8[n], sq[i], tiles, table)
                    o_l = bf.linear_attention_row(q[n], [k[t] for t in comp], [v[t] for t in comp]) \
                        if comp else [0.0] * d
                    al = x.alpha[h].astype(float)
                    out[b, h, n] = [al[c] * o_s[c] + (1 - al[c]) * o_l[c] for c in range(d)]
    return out


@pytest.mark.parametrize("top_k", [0, 2, 5])
def test_forward_fp8_matches_token_brute_force(top_k):
    x = make_custom(1, 2, 70, 150, 8, top_k, dtype="bf16", kind="smooth", seed=5, block=32,
                    scale=3.0)
    got, idx = fp8.forward_fp8(x)
    want = _brute_forward_fp8(x)
    assert np.allclose(got, want, rtol=1e-10, atol=1e-12), np.abs(got - want).max()
    ref_idx = so.route(x)
    assert np.array_equal(idx, ref_idx)


def _e4m3_exact_inputs(n, d, b, top_k, scales=(0.125, 8.0, 8.0)):
    """f32 inputs whose values are E4M3 values and each 64-token block holds the entry 448,
    so that every block scale of either reading is exactly 1."""
    def t(scale):
        x = fp8.e4m3_round(RNG.standard_normal((1, 2, n, d)) * scale)
        for j in range(-(-n // b)):
            x[:, :, j * b, 0] = 448.0
        return x.astype(np.float32)
    pr = Problem(1, 2, n, n, d, b, top_k, "f32", "custom_e4m3")
    pq = (RNG.standard_normal((d, d)) / math.sqrt(d)).astype(np.float32)
    pk = (RNG.standard_normal((d, d)) / math.sqrt(d)).astype(np.float32)
    al = RNG.uniform(0.2, 0.9, (2, d)).astype(np.float32)
    return Inputs(pr, t(scales[0]), t(scales[1]), t(scales[2]), pq, pk, al)


def _p_rounding_bound(x, idx, sub_step):
    """Per element, alpha times the bound on the sparse branch's change from rounding P to
    E4M3: relative 2^-4 per weight in the normal range plus `sub_step` (absolute, relative
    to the row's largest weight) per weight below it, over the row's weight sum."""
    p = x.problem
    out = np.zeros((p.batch, p.heads, p.n_q, p.head_dim))
    for h in range(p.heads):
        q, k, v = (x.as_f64(nm)[0, h] for nm in ("q", "k", "v"))
        for i in range(p.nbq):
            toks = np.concatenate([np.arange(j * p.block, min((j + 1) * p.block, p.n_kv))
                                   for j in idx[0, h, i]])
            rows = np.arange(i * p.block, min((i + 1) * p.block, p.n_q))
            lg = q[rows] @ k[toks].T / math.sqrt(p.head_dim)
            w = np.exp(lg - lg.max(1, keepdims=True))
            bnd = (2.0 ** -4 * (w @ np.abs(v[toks])) + sub_step * np.abs(v[toks]).sum(0)) \
                / w.sum(1, keepdims=True)
            out[0, h, rows] = x.alpha[h].astype(float) * bnd
    return out


def test_forward_fp8_on_exact_inputs_differs_from_forward_only_by_p_rounding():
    x = _e4m3_exact_inputs(192, 16, 64, 2)
    o8, i8 = fp8.forward_fp8(x)
    o, i = so.forward(x)
    assert np.array_equal(i8, i)
    bound = _p_rounding_bound(x, i, 2.0 ** -13)
    assert np.all(np.abs(o8 - o) <= bound + 1e-12)
    assert np.abs(o8 - o).max() > 0


def test_forward_fp8_literal_on_exact_inputs_differs_only_by_p_rounding():
    x = _e4m3_exact_inputs(192, 16, 64, 2)
    o8, i8 = fp8.forward_fp8_literal(x)
    o, i = so.forward(x)
    assert np.array_equal(i8, i)
    bound = _p_rounding_bound(x, i, 2.0 ** -10 / 448.0)
    assert np.all(np.abs(o8 - o) <= bound + 1e-12)
    assert np.abs(o8 - o).max() > 0


def test_literal_scales_are_float32_absmax_over_448():
    x = RNG.standard_normal((64 + 10, 4)).astype(np.float32).astype(np.float64)
    x[3, 1] = -7.0
    x8, s = fp8.quantise_blocks_absmax(x, 64)
    assert s[0] == float(np.float32(7.0 / 448.0)) and s[0] != 2.0 ** -6 * 1.0000001
    assert s[1] == float(np.float32(np.abs(x[64:]).max() / 448.0))
    assert np.abs(x8).max() <= 448.0 and abs(x8[3, 1]) == 448.0
    assert np.array_equal(fp8.e4m3_round(x8), x8)
    z8, zs = fp8.quantise_blocks_absmax(np.zeros((64, 3)), 64)
    assert zs[0] == 1.0 and not z8.any()


def test_literal_equal_logits_give_mean_of_dequantised_v():
    """All logits equal: p = 1 everywhere, s_P = 1/448, P8 = 448 (exact), so O_s is the plain
    mean of the dequantised values, for any number of tiles."""
    d, b = 8, 64
    q8 = fp8.e4m3_round(RNG.standard_normal((64, d)) * 50)
    k8 = np.zeros((2 * b, d))
    v8 = fp8.e4m3_round(RNG.standard_normal((2 * b, d)) * 100)
    sv = np.array([0.25, 0.5])
    o = fp8.sparse_block_fp8_literal(q8, 0.5, k8, np.array([1.0, 1.0]), v8, sv, [0, 1], b)
    want = (0.25 * v8[:b].sum(0) + 0.5 * v8[b:].sum(0)) / (2 * b)
    assert np.allclose(o, want[None], rtol=1e-14, atol=1e-14)


# --------------------------------------------------------------------------- all-heads wrappers
def test_pisa_forward_wrapper_matches_head_function():
    x = make_custom(2, 2, 100, 130, 8, 2, dtype="f32", block=32, seed=9)
    out, idx = pisa.forward(x)
    for b in range(2):
        for h in range(2):
            o, r = pisa.forward_head(x.as_f64("q")[b, h], x.as_f64("k")[b, h],
                                     x.as_f64("v")[b, h], x.proj_q.astype(float),
                                     x.proj_k.astype(float), 32, 2)
            assert np.array_equal(out[b, h], o)
            assert np.array_equal(idx[b, h], r.idx)
    rows = np.array([0, 31, 32, 99])
    out2, _ = pisa.forward(x, heads=[(1, 1)], rows=rows)
    assert np.allclose(out2[1, 1, rows], out[1, 1, rows], rtol=1e-13, atol=1e-15)
    assert np.isnan(out2[0, 0]).all() and np.isnan(np.delete(out2[1, 1], rows, 0)).all()


@pytest.mark.parametrize("router", ["learnable", "taylor"])
def test_route_full_matches_head_functions(router):
    x = make_custom(2, 3, 90, 200, 16, 3, dtype="bf16", block=32, seed=11, kind="smooth")
    res = so.route_full(x, router=router)
    assert len(res) == 2 and all(len(r) == 3 for r in res)
    for b in range(2):
        for h in range(3):
            q, k = x.as_f64("q")[b, h], x.as_f64("k")[b, h]
            if router == "taylor":
                ref = so.route_head_taylor(q, k, 32, 3)
            else:
                ref = so.route_head(q, k, x.proj_q.astype(float), x.proj_k.astype(float), 32, 3)
            got = res[b][h]
            assert np.array_equal(got.idx, ref.idx)
            assert np.array_equal(got.scores, ref.scores)
            assert np.array_equal(got.near_tie, ref.near_tie)
    if router == "learnable":
        assert np.array_equal(np.stack([np.stack([r.idx for r in row]) for row in res]),
                              so.route(x))
