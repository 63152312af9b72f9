"""CPU float64 oracle of the exact-or-approximate (piecewise) attention tail.

TEST INFRASTRUCTURE ONLY (see the package header): imported by the test suite, never by the
GPU library.

Method (PISA page, "Piecewise Sparse Attention", section "Algoritmo Central", the core
algorithm): the key blocks routed to a query block are attended exactly; every other key
block enters the SAME softmax normalisation through a Taylor expansion of exp(q.k) around
the block's centroid k_bar_j:

  exp(tau q.k_n) ~= a_j (1 + tau q.(k_n - k_bar_j)),     a_j = exp(tau q.k_bar_j)

Summed over the block's valid tokens n (n_j of them):

  numerator   sum_n exp(tau q.k_n) v_n ~= a_j (Vsum_j + tau q H_j),
              Vsum_j = sum_n v_n,   H_j = sum_n (k_n - k_bar_j)^T v_n   (d x d);
  denominator sum_n exp(tau q.k_n)     ~= a_j n_j   (the first-order term is
              tau q . sum_n (k_n - k_bar_j) = 0, because the deviations from the block
              mean sum to zero).

The zero-order part is kept per block; the first-order part uses one global matrix H_bar,
the mean of H_j over ALL key blocks of the head, instead of each block's H_j. So for query
token t of query block i, with S = sel(i) and U = the other key blocks:

  N_t = sum_{j in S} sum_n e^{tau q_t.k_n} v_n + sum_{j in U} a_tj Vsum_j
        + tau (q_t H_bar) sum_{j in U} a_tj
  D_t = sum_{j in S} sum_n e^{tau q_t.k_n}     + sum_{j in U} a_tj n_j
  o_t = N_t / D_t

Readings (the page prints N_t but not D_t and gives no scale): tau = 1/sqrt(d), the scale
of the exact branch, multiplies every exponent and the first-order term (the page folds it
into q); D_t is the expansion above, whose first-order part vanishes; n_j and the centroid
count only a partial last block's valid tokens; H_bar averages over every key block,
selected or not; the routed set S comes from the same router as the SLA2 forward (SLA2
page, section 2.B); nothing is mixed afterwards (no alpha: the page merges the two parts
inside one normalisation instead of adding branch outputs).
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

from .sla_oracle import (_head, block_slice, n_blocks, pool_blocks, route_head,
                         route_head_taylor)


def block_stats(k: np.ndarray, v: np.ndarray, block: int):
    """Per key block j: centroid k_bar_j (mean of the valid keys), Vsum_j, n_j and the
    first-order matrix H_j = sum_n (k_n - k_bar_j)^T v_n (rows: key channel, columns: value
    channel). Returns (k_bar [nb, d], vsum [nb, d], counts [nb], H [nb, d, d])."""
    n, d = k.shape
    nb = n_blocks(n, block)
    k_bar = pool_blocks(k, block)
    vsum = np.empty((nb, d))
    counts = np.empty(nb)
    H = np.empty((nb, d, d))
    for j in range(nb):
        sl = block_slice(j, n, block)
        vsum[j] = v[sl].sum(axis=0)
        counts[j] = sl.stop - sl.start
        H[j] = (k[sl] - k_bar[j]).T @ v[sl]
    return k_bar, vsum, counts, H


def tail_rows(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, sel: Sequence[int],
              k_bar: np.ndarray, vsum: np.ndarray, counts: np.ndarray, H_bar: np.ndarray,
              block: int) -> np.ndarray:
    """o_t = N_t / D_t for some query rows of one query block (definitions in the header).
    All exponentials share one per-row maximum over the exact logits and the centroid
    logits."""
    n, d = k.shape
    tau = 1.0 / math.sqrt(d)
    nb = k_bar.shape[0]
    sel = np.asarray(sel, dtype=np.int64)
    uns = np.setdiff1d(np.arange(nb), sel)
    if sel.size:
        toks = np.concatenate([np.arange(n)[block_slice(j, n, block)] for j in sel])
        z_e = tau * (q_rows @ k[toks].T)
    else:
        toks = np.zeros(0, dtype=np.int64)
        z_e = np.zeros((q_rows.shape[0], 0))
    z_u = tau * (q_rows @ k_bar[uns].T)
    m = np.concatenate([z_e, z_u], axis=1).max(axis=1, keepdims=True)
    w_e = np.exp(z_e - m)
    a_u = np.exp(z_u - m)
    num = w_e @ v[toks] + a_u @ vsum[uns] + tau * (q_rows @ H_bar) * a_u.sum(axis=1)[:, None]
    den = w_e.sum(axis=1) + a_u @ counts[uns]
    return num / den[:, None]


def forward_head(q, k, v, proj_q, proj_k, block: int, top_k: int,
                 rows: Optional[np.ndarray] = None, router: str = "learnable"):
    """Piecewise forward of one (b, h). Returns (out [Nq, d], Route). ``rows``: optional
    query-token indices to evaluate (NaN elsewhere); the router always runs in full."""
    nq, d = q.shape
    if router == "taylor":
        r = route_head_taylor(q, k, block, top_k)
    else:
        r = route_head(q, k, proj_q, proj_k, block, top_k)
    k_bar, vsum, counts, H = block_stats(k, v, block)
    H_bar = H.mean(axis=0)
    out = np.full((nq, d), np.nan)
    want = np.arange(nq) if rows is None else np.asarray(rows)
    for i in np.unique(want // block):
        toks = np.arange(nq)[block_slice(i, nq, block)]
        toks = toks[np.isin(toks, want)]
        out[toks] = tail_rows(q[toks], k, v, r.idx[i], k_bar, vsum, counts, H_bar, block)
    return out, r


def forward(inputs, heads: Optional[Sequence[tuple]] = None,
            rows: Optional[np.ndarray] = None):
    """Piecewise forward (learnable router) for all or selected (b, h) pairs.
    Returns (out [B, H, Nq, d] float64, NaN where not evaluated; idx [B, H, Nbq, k])."""
    p = inputs.problem
    pq = inputs.proj_q.astype(np.float64)
    pk = inputs.proj_k.astype(np.float64)
    out = np.full((p.batch, p.heads, p.n_q, p.head_dim), np.nan)
    idx = np.full((p.batch, p.heads, p.nbq, p.top_k), -1, np.int32)
    pairs = heads if heads is not None else [(b, h) for b in range(p.batch) for h in range(p.heads)]
    for b, h in pairs:
        o, r = forward_head(_head(inputs, "q", b, h), _head(inputs, "k", b, h),
                            _head(inputs, "v", b, h), pq, pk, p.block, p.top_k, rows)
        out[b, h] = o
        idx[b, h] = r.idx
    return out, idx
