"""CPU float64 oracle for the quantised sparse branch (OCP FP8 E4M3FN).

TEST INFRASTRUCTURE ONLY (see ``oracle.sla_oracle``).

SLA2 page, section 2.C: the sparse branch is quantised to low precision (INT8 or FP8) and
the forward pass uses the quantised attention. The router, the linear branch and the mix
are unquantised, exactly as in ``sla_oracle``.

Readings (the pages give no format details; the fp8 workload asks for per-64x128-block
absmax scales on Q K^T and a per-tile scale on P.V):
* Format: OCP E4M3FN (bias 7, 3 mantissa bits, finite max 448, no infinities, one NaN
  pattern per sign). Rounding: to nearest, ties to even, saturating at +-448.
* Q, K and V are quantised per (b, h, 64-token block) with a power-of-two scale derived
  from the block's absolute maximum over its valid tokens and all channels (an E8M0 block
  scale): s = 2^e with e the smallest integer such that 448 * 2^e >= absmax (e = 0 when
  the block is all zero); x8 = E4M3(x * 2^-e), which is an exact scaling followed by one
  rounding; the dequantised value is x8 * s.
* Logits of a (query block i, key tile j) pair: z = s_Q(i) s_K(j) (Q8_i K8_j^T) / sqrt(d);
  y = z * log2(e) (base-2 units).
* P is quantised per key tile and query row: with T = floor(max over the tile's keys of y),
  P8 = E4M3(2^7 * 2^(y - T)) (values in (0, 256), the row's largest in [128, 256)), and the
  tile contributes 2^(T - 7) * s_V(j) * (P8 V8_j): every per-row weight is a power of two.
* O_s = sum_j 2^(T_j - 7) s_V(j) (P8_j V8_j) / sum_j sum_keys 2^y: the normaliser uses the
  unquantised probabilities.
This form does not depend on the order in which tiles are visited: an online softmax that
keeps its running maximum on integers and rescales by exact powers of two gives the same
value in exact arithmetic.

A second, literal reading of the fp8 workload's wording is kept beside it for comparison
(``forward_fp8_literal``): float32 absmax/448 block scales for Q, K and V, and one
absmax/448 scale for P over each 64 x 64 (query block x key tile) tile of the online
softmax, visited in ascending key-block order. The GPU path implements the first reading;
the second only measures how far the choice of reading moves the output.
"""
from __future__ import annotations

import math
from typing import Sequence

import numpy as np

from .sla_oracle import (block_slice, linear_complement, mix, n_blocks, route_head,
                         selection_mask, block_summaries, _head)

E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each 8-bit E4M3FN code (OCP 8-bit floating point specification)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def e4m3_round(x: np.ndarray) -> np.ndarray:
    """Nearest E4M3FN value, ties to even, saturating at +-448 (NaN stays NaN).

    Normal numbers with leading exponent E carry 3 fraction bits, so their spacing is
    2^(E-3); below 2^-6 the spacing is the subnormal step 2^-9.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)                    # a = f * 2^e, f in [0.5, 1)
    lead = np.maximum(e - 1, -6)
    step = np.exp2(lead - 3.0)
    r = np.rint(a / step) * step          # rint: ties to even
    r = np.minimum(r, E4M3_MAX)
    return np.where(np.isnan(x), np.nan, np.copysign(r, x))


def block_scale_exponent(amax: float) -> int:
    """Smallest integer e with 448 * 2^e >= amax (0 for an all-zero block)."""
    if amax == 0:
        return 0
    _, ex = math.frexp(amax / E4M3_MAX)      # amax/448 = f * 2^ex, f in [0.5, 1)
    e = ex
    while E4M3_MAX * math.ldexp(1.0, e - 1) >= amax:   # exact comparisons (powers of two)
        e -= 1
    while E4M3_MAX * math.ldexp(1.0, e) < amax:
        e += 1
    return e


def quantise_blocks(x: np.ndarray, block: int):
    """Per-block E4M3 quantisation of one (b, h) tensor x [N, d] (float64 holding the exact
    stored values). Returns (x8 values [N, d] float64, s [Nb] float64 powers of two)."""
    n = x.shape[0]
    nb = n_blocks(n, block)
    x8 = np.empty_like(x)
    s = np.empty(nb)
    for j in range(nb):
        sl = block_slice(j, n, block)
        e = block_scale_exponent(float(np.abs(x[sl]).max()))
        x8[sl] = e4m3_round(x[sl] * math.ldexp(1.0, -e))
        s[j] = math.ldexp(1.0, e)
    return x8, s


def sparse_rows_fp8(q8_rows: np.ndarray, sq: float, k8: np.ndarray, sk: np.ndarray,
                    v8: np.ndarray, sv: np.ndarray, sel: Sequence[int], block: int) -> np.ndarray:
    """Quantised sparse attention of some query rows of one query block (module readings)."""
    n, d = k8.shape
    if len(sel) == 0:
        return np.zeros((q8_rows.shape[0], d))
    tau = 1.0 / math.sqrt(d)
    log2e = 1.0 / math.log(2.0)
    ys, Ts = [], []
    for j in sel:
        sl = block_slice(j, n, block)
        y = sq * sk[j] * tau * (q8_rows @ k8[sl].T) * log2e
        ys.append(y)
        Ts.append(np.floor(y.max(axis=1)))
    G = np.max(np.stack(Ts, axis=1), axis=1)         # common reference, avoids overflow
    num = np.zeros((q8_rows.shape[0], d))
    den = np.zeros(q8_rows.shape[0])
    for j, y, T in zip(sel, ys, Ts):
        sl = block_slice(j, n, block)
        p8 = e4m3_round(np.exp2(7.0 + y - T[:, None]))
        num += (np.exp2(T - 7.0 - G) * sv[j])[:, None] * (p8 @ v8[sl])
        den += np.exp2(y - G[:, None]).sum(axis=1)
    return num / den[:, None]


def forward_fp8(inputs, heads=None, rows=None):
    """SLA2 forward with the quantised sparse branch. Returns (out, idx) like
    ``sla_oracle.forward``; NaN where not evaluated."""
    p = inputs.problem
    pq = inputs.proj_q.astype(np.float64)
    pk = inputs.proj_k.astype(np.float64)
    al = inputs.alpha.astype(np.float64)
    out = np.full((p.batch, p.heads, p.n_q, p.head_dim), np.nan)
    idx = np.full((p.batch, p.heads, p.nbq, p.top_k), -1, np.int32)
    pairs = heads if heads is not None else [(b, h) for b in range(p.batch) for h in range(p.heads)]
    for b, h in pairs:
        q = _head(inputs, "q", b, h)
        k = _head(inputs, "k", b, h)
        v = _head(inputs, "v", b, h)
        r = route_head(q, k, pq, pk, p.block, p.top_k)
        M = selection_mask(r.idx, p.nbk)
        S, z = block_summaries(k, v, p.block)
        q8, sq = quantise_blocks(q, p.block)
        k8, sk = quantise_blocks(k, p.block)
        v8, sv = quantise_blocks(v, p.block)
        want = np.arange(p.n_q) if rows is None else np.asarray(rows)
        for i in np.unique(want // p.block):
            toks = np.arange(p.n_q)[block_slice(i, p.n_q, p.block)]
            toks = toks[np.isin(toks, want)]
            o_s = sparse_rows_fp8(q8[toks], sq[i], k8, sk, v8, sv, r.idx[i], p.block)
            o_l = linear_complement(q[toks], S, z, M[i])
            out[b, h, toks] = mix(al[h], o_s, o_l)
        idx[b, h] = r.idx
    return out, idx


# ----------------------------------------------------------------------------- literal reading
def quantise_blocks_absmax(x: np.ndarray, block: int):
    """Per-block E4M3 quantisation with a float32 scale s = fp32(absmax / 448) (s = 1 for an
    all-zero block) and x8 = E4M3(fp32(x / s)): the scale is not a power of two, so the
    division is rounded to float32 before the E4M3 rounding. x: [N, d] float64 holding
    float32-exact values. Returns (x8 [N, d] float64, s [Nb] float64)."""
    n = x.shape[0]
    nb = n_blocks(n, block)
    x8 = np.empty_like(x)
    s = np.empty(nb)
    for j in range(nb):
        sl = block_slice(j, n, block)
        amax = float(np.abs(x[sl]).max())
        sj = np.float32(amax / E4M3_MAX) if amax > 0 else np.float32(1.0)
        x8[sl] = e4m3_round((x[sl].astype(np.float32) / sj).astype(np.float64))
        s[j] = float(sj)
    return x8, s


def sparse_block_fp8_literal(q8_blk: np.ndarray, sq: float, k8: np.ndarray, sk: np.ndarray,
                             v8: np.ndarray, sv: np.ndarray, sel: Sequence[int],
                             block: int) -> np.ndarray:
    """Quantised sparse attention of all rows of one query block, literal reading: online
    softmax over the selected key tiles in ascending order with m the running row maximum
    of the logits z = tau s_Q s_K (Q8 K8^T), p = exp(z - m_new), one scale
    s_P = max(p over the query block x key tile) / 448 per tile, P8 = E4M3(p / s_P),
    acc <- acc e^(m - m_new) + s_P s_V (P8 V8), l <- l e^(m - m_new) + sum p (unquantised)."""
    n, d = k8.shape
    rows = q8_blk.shape[0]
    if len(sel) == 0:
        return np.zeros((rows, d))
    tau = 1.0 / math.sqrt(d)
    m = np.full(rows, -np.inf)
    acc = np.zeros((rows, d))
    lsum = np.zeros(rows)
    for j in sorted(sel):
        sl = block_slice(j, n, block)
        z = tau * sq * sk[j] * (q8_blk @ k8[sl].T)
        m_new = np.maximum(m, z.max(axis=1))
        corr = np.exp(m - m_new)
        p = np.exp(z - m_new[:, None])
        s_p = p.max() / E4M3_MAX
        p8 = e4m3_round(p / s_p)
        acc = acc * corr[:, None] + (s_p * sv[j]) * (p8 @ v8[sl])
        lsum = lsum * corr + p.sum(axis=1)
        m = m_new
    return acc / lsum[:, None]


def forward_fp8_literal(inputs, heads=None, rows=None):
    """SLA2 forward with the quantised sparse branch in the literal reading (module
    docstring); router, linear branch and mix as in ``forward_fp8``. Returns (out, idx)."""
    p = inputs.problem
    pq = inputs.proj_q.astype(np.float64)
    pk = inputs.proj_k.astype(np.float64)
    al = inputs.alpha.astype(np.float64)
    out = np.full((p.batch, p.heads, p.n_q, p.head_dim), np.nan)
    idx = np.full((p.batch, p.heads, p.nbq, p.top_k), -1, np.int32)
    pairs = heads if heads is not None else [(b, h) for b in range(p.batch) for h in range(p.heads)]
    for b, h in pairs:
        q = _head(inputs, "q", b, h)
        k = _head(inputs, "k", b, h)
        v = _head(inputs, "v", b, h)
        r = route_head(q, k, pq, pk, p.block, p.top_k)
        M = selection_mask(r.idx, p.nbk)
        S, z = block_summaries(k, v, p.block)
        q8, sq = quantise_blocks_absmax(q, p.block)
        k8, sk = quantise_blocks_absmax(k, p.block)
        v8, sv = quantise_blocks_absmax(v, p.block)
        want = np.arange(p.n_q) if rows is None else np.asarray(rows)
        for i in np.unique(want // p.block):
            blk = np.arange(p.n_q)[block_slice(i, p.n_q, p.block)]
            o_blk = sparse_block_fp8_literal(q8[blk], sq[i], k8, sk, v8, sv, r.idx[i], p.block)
            keep = np.isin(blk, want)
            toks = blk[keep]
            o_l = linear_complement(q[toks], S, z, M[i])
            out[b, h, toks] = mix(al[h], o_blk[keep], o_l)
        idx[b, h] = r.idx
    return out, idx
