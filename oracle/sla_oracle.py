"""CPU float64 oracle for SLA2 sparse-linear attention (forward).

TEST INFRASTRUCTURE ONLY. Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The GPU library never
does, and shares no code with it.

What is computed (per batch b and head h, independently):

* Mix (SLA2 page, section 2.A, "Formulação de Mistura"): O = alpha (.) O_s + (1 - alpha) (.) O_l,
  alpha a per-channel ratio vector.
* Router (SLA2 page, section 2.B, "Roteador Aprendível"): the router reads Q and K only;
  it mean-pools adjacent token blocks, applies the learnable projections proj_q and
  proj_k, and keeps the top-k blocks per query block.
* Sparse branch (SLA2 page, sections 1 and 2.B): exact softmax attention restricted to
  the routed blocks.
* Linear branch (SALAD page, section 2 "Ramos Paralelos": kernel feature map such as
  ReLU, linear cost; SPLA page, section 2.2: the linear term covers exactly the blocks the
  sparse part did not select).
* Training-free router (SPLA page, section 2.1), selectable instead of the learnable one:
  the block score is the second-order Taylor estimate of the block's attention mass
  around its mean key with a diagonal covariance (``taylor_scores``).

Readings taken where the pages are silent:
  block b for queries and keys; pool over valid tokens only; project after pooling with
  x @ P (P stored [d_in, d_out]); plain dot-product block score; ties broken toward the
  lowest key-block index; softmax scale 1/sqrt(d); phi = ReLU on raw Q and K; eps = 1e-6
  added to the linear denominator; top_k = 0 gives O_s = 0; an empty complement gives
  O_l = 0.

Everything is float64 on values upcast exactly from the stored input bits.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

EPS = 1e-6


def relu(x: np.ndarray) -> np.ndarray:
    """Feature map of the linear branch (SALAD page, section 2: ReLU kernel)."""
    return np.maximum(x, 0.0)


def n_blocks(n: int, block: int) -> int:
    return -(-n // block)


def block_slice(j: int, n: int, block: int) -> slice:
    """Token range of block j: [j*b, min((j+1)*b, n))."""
    return slice(j * block, min((j + 1) * block, n))


# ----------------------------------------------------------------------------- router
def pool_blocks(x: np.ndarray, block: int) -> np.ndarray:
    """Mean over each block of adjacent tokens, valid tokens only.

    SLA2 page, section 2.B (the router pools adjacent token blocks by their mean).
    x: [N, d] float64 -> [ceil(N/b), d].
    """
    n = x.shape[0]
    return np.stack([x[block_slice(j, n, block)].mean(axis=0) for j in range(n_blocks(n, block))])


def project(pooled: np.ndarray, proj: np.ndarray) -> np.ndarray:
    """Learnable projection of pooled vectors (SLA2 page, section 2.B): pooled @ proj."""
    return pooled @ proj


def block_scores(q_tilde: np.ndarray, k_tilde: np.ndarray) -> np.ndarray:
    """Block relevance score s_ij = q~_i . k~_j (SLA2 page, section 2.B)."""
    return q_tilde @ k_tilde.T


def select_topk(scores: np.ndarray, top_k: int) -> np.ndarray:
    """Top-k key blocks per query-block row, ties to the lowest index, ascending output.

    SLA2 page, section 2.B: keep the top-k pooled weights. Ordering key (-s_ij, j).
    Returns int32 [rows, top_k].
    """
    rows, nbk = scores.shape
    out = np.empty((rows, top_k), dtype=np.int32)
    j = np.arange(nbk)
    for i in range(rows):
        order = np.lexsort((j, -scores[i]))    # primary -s, secondary j
        out[i] = np.sort(order[:top_k])
    return out


def boundary_gaps(scores: np.ndarray, top_k: int) -> np.ndarray:
    """Per row, s_(k) - s_(k+1) in descending order (inf when k is 0 or all blocks)."""
    rows, nbk = scores.shape
    if top_k == 0 or top_k >= nbk:
        return np.full(rows, np.inf)
    srt = -np.sort(-scores, axis=1)
    return srt[:, top_k - 1] - srt[:, top_k]


NEAR_TIE_REL = 1e-12


def near_ties(scores: np.ndarray, gaps: np.ndarray) -> np.ndarray:
    """Rows whose boundary gap is below 1e-12 of the row's largest |score|: there a rounding
    difference of the score arithmetic (about 1e-16 relative in float64) could decide which
    block is the k-th, so more than one selection may be reported as correct. An exact tie
    (gap 0) is flagged too; a row with an infinite gap (k = 0 or all blocks) never is."""
    scale = np.abs(scores).max(axis=1) if scores.size else np.zeros(scores.shape[0])
    return gaps < NEAR_TIE_REL * scale


@dataclass
class Route:
    idx: np.ndarray        # int32 [Nbq, k], ascending
    scores: np.ndarray     # float64 [Nbq, Nbk]
    gaps: np.ndarray       # float64 [Nbq]
    near_tie: np.ndarray   # bool [Nbq]: gap < 1e-12 * max|s| (a plausible rounding flip)


def route_head(q: np.ndarray, k: np.ndarray, proj_q: np.ndarray, proj_k: np.ndarray,
               block: int, top_k: int) -> Route:
    """Router of one (b, h): pool -> project -> score -> top-k (SLA2 page, section 2.B)."""
    qt = project(pool_blocks(q, block), proj_q)
    kt = project(pool_blocks(k, block), proj_k)
    s = block_scores(qt, kt)
    idx = select_topk(s, top_k)
    gaps = boundary_gaps(s, top_k)
    return Route(idx, s, gaps, near_ties(s, gaps))


# ----------------------------------------------------------------------------- Taylor router
def block_variances(x: np.ndarray, block: int) -> np.ndarray:
    """Per block and channel, the population variance of x over the block's valid tokens
    (the diagonal of the block's key covariance). x: [N, d] -> [ceil(N/b), d]."""
    n = x.shape[0]
    out = []
    for j in range(n_blocks(n, block)):
        xb = x[block_slice(j, n, block)]
        dev = xb - xb.mean(axis=0)
        out.append((dev * dev).mean(axis=0))
    return np.stack(out)


def taylor_scores(q_bar: np.ndarray, k_bar: np.ndarray, k_var: np.ndarray) -> np.ndarray:
    """Training-free block score (SPLA page, section 2.1): the expected exponential
    attention score of a query over a block's keys, expanded to second order around the
    block mean with the covariance taken diagonal, exp(tau q.k_bar)(1 + tau^2 q^T diag(var)
    q / 2), with the attention scale tau = 1/sqrt(d). Returned as its logarithm,
    tau q.k_bar + log1p(tau^2 (q*q).var / 2), which ranks the blocks identically and does not
    overflow. q_bar: [Nq, d] (pooled queries, no projection); k_bar, k_var: [Nk, d]."""
    d = q_bar.shape[1]
    tau = 1.0 / math.sqrt(d)
    return tau * (q_bar @ k_bar.T) + np.log1p(0.5 * tau * tau * ((q_bar * q_bar) @ k_var.T))


def route_head_taylor(q: np.ndarray, k: np.ndarray, block: int, top_k: int) -> Route:
    """Training-free router of one (b, h): pool Q and K (means), block variances of K,
    Taylor score, top-k with the same tie rule and output order as route_head."""
    s = taylor_scores(pool_blocks(q, block), pool_blocks(k, block), block_variances(k, block))
    idx = select_topk(s, top_k)
    gaps = boundary_gaps(s, top_k)
    return Route(idx, s, gaps, near_ties(s, gaps))


def selection_mask(idx: np.ndarray, nbk: int) -> np.ndarray:
    """0/1 matrix M[i, j] = 1 iff key block j is routed to query block i."""
    m = np.zeros((idx.shape[0], nbk), dtype=np.float64)
    for i in range(idx.shape[0]):
        m[i, idx[i]] = 1.0
    return m


# ----------------------------------------------------------------------------- sparse branch
def sparse_rows(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, sel: Sequence[int],
                block: int) -> np.ndarray:
    """Exact softmax attention of some query rows over the tokens of the selected blocks.

    SLA2 page, sections 1 and 2.B (exact attention on the routed positions); scale
    1/sqrt(d). With no selected block the result is 0.
    """
    n, d = k.shape
    if len(sel) == 0:
        return np.zeros((q_rows.shape[0], d))
    toks = np.concatenate([np.arange(n)[block_slice(j, n, block)] for j in sel])
    logits = (q_rows @ k[toks].T) / math.sqrt(d)
    logits -= logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    p /= p.sum(axis=1, keepdims=True)
    return p @ v[toks]


# ----------------------------------------------------------------------------- linear branch
def block_summaries(k: np.ndarray, v: np.ndarray, block: int):
    """Per key block j: S_j = phi(K_j)^T V_j (d x d) and z_j = sum_t phi(K_j)_t (d).

    SALAD page, section 2 (ReLU kernel linear attention, linear cost); SPLA page, section
    2.2 (the linear state is built from key blocks).
    """
    n, d = k.shape
    nb = n_blocks(n, block)
    S = np.empty((nb, d, d))
    z = np.empty((nb, d))
    for j in range(nb):
        fk = relu(k[block_slice(j, n, block)])
        S[j] = fk.T @ v[block_slice(j, n, block)]
        z[j] = fk.sum(axis=0)
    return S, z


def linear_complement(q_rows: np.ndarray, S: np.ndarray, z: np.ndarray,
                      mask_row: np.ndarray) -> np.ndarray:
    """Linear attention of some query rows over the key blocks NOT routed to them.

    SPLA page, section 2.2: the residual linear attention covers only the unselected
    blocks. Computed directly from the complement (1 - M) so that it is independent of the
    total-minus-selected form used on the GPU. O_l = phi(q) S_c / (phi(q) . z_c + eps).
    """
    comp = 1.0 - mask_row                     # [Nbk]
    S_c = np.tensordot(comp, S, axes=(0, 0))  # [d, d]
    z_c = comp @ z                            # [d]
    fq = relu(q_rows)
    return (fq @ S_c) / (fq @ z_c + EPS)[:, None]


# ----------------------------------------------------------------------------- full forward
def mix(alpha_h: np.ndarray, o_s: np.ndarray, o_l: np.ndarray) -> np.ndarray:
    """SLA2 page, section 2.A: O = alpha (.) O_s + (1 - alpha) (.) O_l, per channel."""
    return alpha_h[None, :] * o_s + (1.0 - alpha_h[None, :]) * o_l


@dataclass
class HeadResult:
    out: np.ndarray        # [Nq, d]
    o_s: np.ndarray        # [Nq, d]
    o_l: np.ndarray        # [Nq, d]
    route: Route


def forward_head(q, k, v, proj_q, proj_k, alpha_h, block: int, top_k: int,
                 rows: Optional[np.ndarray] = None, router: str = "learnable") -> HeadResult:
    """SLA2 forward of one (b, h).

    ``rows``: optional query-token indices to evaluate (the router always runs in full);
    unevaluated rows of the returned arrays are NaN. ``router``: "learnable" (SLA2 page,
    section 2.B) or "taylor" (SPLA page, section 2.1; the projections are not used).
    """
    nq, d = q.shape
    nkv = k.shape[0]
    if router == "taylor":
        r = route_head_taylor(q, k, block, top_k)
    else:
        r = route_head(q, k, proj_q, proj_k, block, top_k)
    nbk = n_blocks(nkv, block)
    M = selection_mask(r.idx, nbk)
    S, z = block_summaries(k, v, block)
    o_s = np.full((nq, d), np.nan)
    o_l = np.full((nq, d), np.nan)
    want = np.arange(nq) if rows is None else np.asarray(rows)
    for i in np.unique(want // block):
        toks = np.arange(nq)[block_slice(i, nq, block)]
        toks = toks[np.isin(toks, want)]
        o_s[toks] = sparse_rows(q[toks], k, v, r.idx[i], block)
        o_l[toks] = linear_complement(q[toks], S, z, M[i])
    out = mix(alpha_h, o_s, o_l)
    return HeadResult(out, o_s, o_l, r)


def route(inputs) -> np.ndarray:
    """Block indices for every (b, h): int32 [B, H, Nbq, k]."""
    p = inputs.problem
    q = inputs.as_f64("q")
    k = inputs.as_f64("k")
    pq = inputs.proj_q.astype(np.float64)
    pk = inputs.proj_k.astype(np.float64)
    out = np.empty((p.batch, p.heads, p.nbq, p.top_k), np.int32)
    for b in range(p.batch):
        for h in range(p.heads):
            out[b, h] = route_head(q[b, h], k[b, h], pq, pk, p.block, p.top_k).idx
    return out


def route_full(inputs, router: str = "learnable"):
    """Router results for every (b, h) as a nested list of Route objects."""
    p = inputs.problem
    pq = inputs.proj_q.astype(np.float64)
    pk = inputs.proj_k.astype(np.float64)
    res = []
    for b in range(p.batch):
        row = []
        for h in range(p.heads):
            q = _head(inputs, "q", b, h)
            k = _head(inputs, "k", b, h)
            if router == "taylor":
                row.append(route_head_taylor(q, k, p.block, p.top_k))
            else:
                row.append(route_head(q, k, pq, pk, p.block, p.top_k))
        res.append(row)
    return res


def _head(inputs, name, b, h) -> np.ndarray:
    x = getattr(inputs, name)[b, h]
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def forward(inputs, heads: Optional[Sequence[tuple]] = None,
            rows: Optional[np.ndarray] = None, router: str = "learnable"):
    """SLA2 forward for all (or selected) (b, h) pairs.

    Returns (out [B, H, Nq, d] float64 with NaN where not evaluated, idx [B, H, Nbq, k]).
    ``heads``: optional list of (b, h) pairs to evaluate; ``rows``: optional query rows;
    ``router``: "learnable" or "taylor".
    """
    p = inputs.problem
    pq = inputs.proj_q.astype(np.float64)
    pk = inputs.proj_k.astype(np.float64)
    al = inputs.alpha.astype(np.float64)
    out = np.full((p.batch, p.heads, p.n_q, p.head_dim), np.nan)
    idx = np.full((p.batch, p.heads, p.nbq, p.top_k), -1, np.int32)
    pairs = heads if heads is not None else [(b, h) for b in range(p.batch) for h in range(p.heads)]
    for b, h in pairs:
        r = forward_head(_head(inputs, "q", b, h), _head(inputs, "k", b, h),
                         _head(inputs, "v", b, h), pq, pk, al[h], p.block, p.top_k, rows,
                         router)
        out[b, h] = r.out
        idx[b, h] = r.route.idx
    return out, idx
