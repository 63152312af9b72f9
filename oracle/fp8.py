"""CPU float64 oracle for the quantised sparse branch (OCP FP8 E4M3FN).

TEST INFRASTRUCTURE ONLY (see ``oracle.sla_oracle``).

SLA2 page, section 2.C: the sparse branch is quantised to low precision (INT8 or FP8) and
the forward pass uses the quantised attention. The router, the linear branch and the mix
are unquantised, exactly as in ``sla_oracle``.

Readings (the pages give no format details):
* Format: OCP E4M3FN (bias 7, 3 mantissa bits, finite max 448, no infinities, one NaN
  pattern per sign). Rounding: to nearest, ties to even, saturating at +-448.
* Q, K and V are quantised per (b, h, 64-token block) with the block's absolute maximum
  over its valid tokens and all channels: r = fp32(448 / absmax), s = fp32(absmax / 448)
  (r = s = 1 when absmax is 0); x8 = E4M3(fp32(x * r)); the dequantised value is x8 * s.
* Logits of a (query block i, key block j) tile: z = s_Q(i) s_K(j) (Q8_i K8_j^T) / sqrt(d).
* P is quantised per key tile and query row: with t the row's largest logit inside the
  tile, P8 = E4M3(448 * exp(z - t)) and the row's dequantisation weight for that tile is
  exp(t - m)/448, where m is the row's largest logit over all selected tiles. The tile's
  largest element therefore maps exactly to 448.
* O_s = sum_j exp(t_j - m)/448 * s_V(j) * (P8_j V8_j) / sum_j sum_keys exp(z - m): the
  normaliser uses the unquantised probabilities.
This form does not depend on the order in which tiles are visited: an online softmax that
visits the selected tiles in any order and rescales by exp(m_old - m_new) gives the same
value in exact arithmetic.
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


def f32(x):
    """Round to IEEE binary32 (numpy float32 arithmetic is correctly rounded)."""
    return np.float32(x)


def quantise_blocks(x: np.ndarray, block: int):
    """Per-block E4M3 quantisation of one (b, h) tensor x [N, d] (float64 holding fp32-exact
    values). Returns (x8 values [N, d] float64, s [Nb] float64)."""
    n = x.shape[0]
    nb = n_blocks(n, block)
    x8 = np.empty_like(x)
    s = np.empty(nb)
    for j in range(nb):
        sl = block_slice(j, n, block)
        amax = np.float32(np.abs(x[sl]).max())
        if amax == 0:
            r32, s32 = np.float32(1.0), np.float32(1.0)
        else:
            r32 = f32(np.float32(E4M3_MAX) / amax)
            s32 = f32(amax / np.float32(E4M3_MAX))
        scaled = (x[sl].astype(np.float32) * r32).astype(np.float32)   # fp32 product
        x8[sl] = e4m3_round(scaled.astype(np.float64))
        s[j] = float(s32)
    return x8, s


def sparse_rows_fp8(q8_rows: np.ndarray, sq: float, k8: np.ndarray, sk: np.ndarray,
                    v8: np.ndarray, sv: np.ndarray, sel: Sequence[int], block: int) -> np.ndarray:
    """Quantised sparse attention of some query rows of one query block (module readings)."""
    n, d = k8.shape
    if len(sel) == 0:
        return np.zeros((q8_rows.shape[0], d))
    tau = 1.0 / math.sqrt(d)
    z_tiles = []
    for j in sel:
        sl = block_slice(j, n, block)
        z_tiles.append(sq * sk[j] * tau * (q8_rows @ k8[sl].T))
    m = np.max(np.stack([zt.max(axis=1) for zt in z_tiles], axis=1), axis=1)   # [rows]
    num = np.zeros((q8_rows.shape[0], d))
    den = np.zeros(q8_rows.shape[0])
    for j, zt in zip(sel, z_tiles):
        sl = block_slice(j, n, block)
        t = zt.max(axis=1)
        p8 = e4m3_round(E4M3_MAX * np.exp(zt - t[:, None]))
        w = np.exp(t - m) / E4M3_MAX
        num += (w * sv[j])[:, None] * (p8 @ v8[sl])
        den += np.exp(zt - m[:, None]).sum(axis=1)
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
