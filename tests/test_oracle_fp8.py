"""Pins of the quantised (E4M3) part of the oracle.

The E4M3FN encoder and decoder are pinned to facts of the OCP 8-bit floating point format
(extreme values, NaN codes, value count, monotonicity) and to a brute-force nearest-value
search over the decoded code table. The quantised sparse branch is pinned by special cases
whose result is known in closed form.
"""
import math

import numpy as np
import pytest

from oracle import fp8
from oracle import sla_oracle as so

RNG = np.random.default_rng(77)


def test_e4m3_decode_table_facts():
    vals = fp8.e4m3_decode(np.arange(256))
    assert vals[0x7E] == 448.0 and vals[0xFE] == -448.0          # largest finite
    assert vals[0x01] == 2.0 ** -9 and vals[0x08] == 2.0 ** -6   # min subnormal, min normal
    assert vals[0x07] == 7 * 2.0 ** -9                            # largest subnormal
    assert vals[0x38] == 1.0 and vals[0x40] == 2.0
    assert np.isnan(vals[0x7F]) and np.isnan(vals[0xFF])
    assert np.isnan(vals).sum() == 2
    assert vals[0x00] == 0.0 and vals[0x80] == 0.0 and math.copysign(1, vals[0x80]) == -1
    pos = vals[:0x7F]
    assert np.all(np.diff(pos) > 0)                               # codes ordered by value
    assert np.array_equal(vals[0x80:0xFF], -pos)
    assert np.unique(vals[~np.isnan(vals)]).size == 253


def _nearest_by_search(x, table_vals, table_codes):
    """Brute force: nearest finite value, ties to the even code, clamp beyond 448."""
    out = np.empty_like(x)
    for n, v in enumerate(x):
        if np.isnan(v):
            out[n] = np.nan
            continue
        vv = min(max(v, -448.0), 448.0)
        dist = np.abs(table_vals - vv)
        best = np.flatnonzero(dist == dist.min())
        if best.size > 1:
            best = [b for b in best if table_codes[b] % 2 == 0]
        out[n] = table_vals[best[0]]
    return out


def test_e4m3_round_is_nearest_even_saturating():
    codes = np.arange(256)
    vals = fp8.e4m3_decode(codes)
    keep = ~np.isnan(vals)
    tv, tc = vals[keep], codes[keep]
    # exact midpoints, values just around them, random values over all binades, and overflow
    mids = (np.sort(np.unique(tv))[1:] + np.sort(np.unique(tv))[:-1]) / 2
    x = np.concatenate([
        mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf),
        RNG.standard_normal(4000) * np.exp2(RNG.integers(-12, 10, 4000)),
        [0.0, -0.0, 448.0, 449.0, 463.99, 464.0, 500.0, 1e30, -1e30, np.nan],
    ]).astype(np.float32).astype(np.float64)
    got = fp8.e4m3_round(x)
    want = _nearest_by_search(x, tv, tc)
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all(), x[~same][:10]


def test_block_scale_exponent_closed_form():
    """e is the smallest integer with 448 * 2^e >= absmax."""
    cases = {448.0: 0, 449.0: 1, 224.0: -1, 224.5: 0, 896.0: 1, 1.0: -8, 1.75: -8,
             1.7500001: -7, 3.5: -7, 0.0: 0, 448.0 * 2.0 ** -20: -20}
    for amax, e in cases.items():
        assert fp8.block_scale_exponent(amax) == e, amax


def test_quantise_blocks_scales_and_bounds():
    x = RNG.standard_normal((3 * 64 + 10, 16)).astype(np.float32).astype(np.float64)
    x[70, 3] = -9.5                                               # block 1 absmax
    x8, s = fp8.quantise_blocks(x, 64)
    assert s.shape == (4,)
    assert s[1] == 2.0 ** -5                                      # 448/64 = 7 < 9.5 <= 14
    assert x8[70, 3] == -320.0      # 9.5 * 32 = 304: midway between 288 and 320, ties to even
    for j in range(4):
        sl = so.block_slice(j, x.shape[0], 64)
        e = np.log2(s[j])
        assert e == int(e)                                        # power of two
        amax = np.abs(x[sl]).max()
        assert 224.0 < amax / s[j] <= 448.0                       # smallest such power
        assert np.array_equal(fp8.e4m3_round(x8[sl]), x8[sl])     # every code is E4M3
        err = np.abs(x8[sl] * s[j] - x[sl])                       # half a step, relative
        assert np.all(err <= np.abs(x[sl]) * 2.0 ** -4 + 2.0 ** -10 * s[j] + 1e-12)
    z8, zs = fp8.quantise_blocks(np.zeros((64, 4)), 64)
    assert zs[0] == 1.0 and not z8.any()


def test_fp8_equal_logits_give_mean_of_dequantised_v():
    """A tile whose logits are all equal has P8 = 128 everywhere (T = 0), so O_s is the
    plain mean of the dequantised values."""
    d, b = 8, 64
    q8 = fp8.e4m3_round(RNG.standard_normal((4, d)) * 50)
    k8 = np.zeros((b, d))
    v8 = fp8.e4m3_round(RNG.standard_normal((b, d)) * 100)
    o = fp8.sparse_rows_fp8(q8, 0.5, k8, np.array([1.0]), v8, np.array([0.25]), [0], b)
    assert np.allclose(o, 0.25 * v8.mean(axis=0)[None], rtol=1e-14, atol=1e-15)


def test_fp8_two_keys_ln2_apart():
    """Logits ln 2 apart give p = (1, 1/2): 128 and 64 after scaling, both exact in E4M3,
    so the output is the exact 2/3 : 1/3 average of the dequantised values."""
    d = 4
    tau = 1 / math.sqrt(d)
    target = math.log(2.0)
    q8 = np.array([[1.0, 0.0, 0.0, 0.0]])
    sk = target / tau          # logits exactly 0 and -ln 2 with k8 = 0 and -1
    k8 = np.zeros((2, d))
    k8[1, 0] = -1.0
    v8 = np.array([[3.0, 1.0, 0.0, 2.0], [0.5, -1.0, 4.0, 2.0]])
    o = fp8.sparse_rows_fp8(q8, 1.0, k8, np.array([sk]), v8, np.array([1.0]), [0], 2)
    assert np.allclose(o[0], (2 * v8[0] + v8[1]) / 3, rtol=1e-14)


def test_fp8_identity_quantisation_within_p_rounding_bound():
    """With E4M3-exact inputs whose block absmax is 448 every scale is 1, the logits are the
    exact ones, and the only difference to exact attention comes from rounding P to E4M3:
    at most 2^-4 of sum p|v| / sum p (plus the subnormal step for p below 2^-13)."""
    d, b, n = 16, 64, 256
    def exact_block(shape, scale):
        x = fp8.e4m3_round(RNG.standard_normal(shape) * scale)
        for j in range(shape[0] // b):
            x[j * b, 0] = 448.0
        return x
    q = exact_block((n, d), 0.125)
    k = exact_block((n, d), 8)
    v = exact_block((n, d), 8)
    q8, sq = fp8.quantise_blocks(q, b)
    k8, sk = fp8.quantise_blocks(k, b)
    v8, sv = fp8.quantise_blocks(v, b)
    assert np.all(sq == 1) and np.all(sk == 1) and np.all(sv == 1)
    assert np.array_equal(q8, q) and np.array_equal(k8, k) and np.array_equal(v8, v)
    sel = [0, 2, 3]
    o8 = fp8.sparse_rows_fp8(q8[:b], 1.0, k8, sk, v8, sv, sel, b)
    ex = so.sparse_rows(q[:b], k, v, sel, b)
    toks = np.concatenate([np.arange(j * b, (j + 1) * b) for j in sel])
    lg = q[:b] @ k[toks].T / math.sqrt(d)
    p = np.exp(lg - lg.max(1, keepdims=True))
    bound = (2.0 ** -4 * (p @ np.abs(v[toks])) + 2.0 ** -13 * np.abs(v[toks]).sum(0).max()) \
        / p.sum(1, keepdims=True)
    assert np.all(np.abs(o8 - ex) <= bound + 1e-12)
    assert np.abs(o8 - ex).max() > 0          # P rounding does act


def test_fp8_visit_order_free_definition_matches_online_form():
    """The order-free definition equals an online softmax (written out independently here)
    that keeps an integer running maximum and rescales by exact powers of two, visiting the
    tiles in ascending or in descending order."""
    d, b = 8, 64
    q8 = fp8.e4m3_round(RNG.standard_normal((8, d)) * 30)
    k8 = fp8.e4m3_round(RNG.standard_normal((4 * b, d)) * 30)
    v8 = fp8.e4m3_round(RNG.standard_normal((4 * b, d)) * 30)
    sk = np.array([2.0 ** -6, 2.0 ** -5, 2.0 ** -7, 2.0 ** -4])
    sv = np.array([0.125, 0.25, 0.5, 1.0])
    sq, sel = 2.0 ** -5, [0, 1, 3]
    got = fp8.sparse_rows_fp8(q8, sq, k8, sk, v8, sv, sel, b)
    for order in (sel, sel[::-1]):
        m = np.full(8, -np.inf)
        acc = np.zeros((8, d))
        lsum = np.zeros(8)
        for j in order:
            y = sq * sk[j] / math.sqrt(d) * (q8 @ k8[j * b:(j + 1) * b].T) / math.log(2)
            T = np.floor(y.max(1))
            mn = np.maximum(m, np.ceil(y.max(1)))
            c = np.exp2(m - mn)
            p8 = fp8.e4m3_round(np.exp2(7 + y - T[:, None]))
            acc = acc * c[:, None] + (np.exp2(T - 7 - mn) * sv[j])[:, None] * (p8 @ v8[j * b:(j + 1) * b])
            lsum = lsum * c + np.exp2(y - mn[:, None]).sum(1)
            m = mn
        assert np.allclose(got, acc / lsum[:, None], rtol=1e-12, atol=1e-14)
