"""CPU float64 oracle of the gradients of the SLA2 forward at a given block selection.

TEST INFRASTRUCTURE ONLY (see ``oracle.sla_oracle``): imported by tests/, never by the GPU
library, and sharing no code with it.

Training (SLA2 page, section 2.B): the router's hard top-k is what the forward uses; for
training the page replaces it by a SoftTop-k, for which it prints no formula. This oracle
therefore differentiates the forward at a FIXED selection: no gradient flows into proj_q or
proj_k through the top-k (the SoftTop-k gradient is parity unpinned). Section 2.C: the
forward may run the quantised attention while the backward stays in higher precision; this
oracle differentiates the unquantised forward of ``sla_oracle`` in float64.

For one (b, h), query block i with rows R_i, selected tokens T_i, complement tokens C_i,
tau = 1/sqrt(d), phi = ReLU (derivative 1 for x > 0, 0 otherwise) and an upstream gradient
dO of the output:
  mix:     dalpha = sum_n dO[n] (.) (O_s[n] - O_l[n]);  dO_s = alpha dO,  dO_l = (1-alpha) dO
  sparse:  P = softmax_{m in T_i}(tau q_n . k_m),  dV_m += sum_n P_nm dO_s[n],
           dP_nm = dO_s[n] . v_m,  dS_nm = P_nm (dP_nm - sum_m' P_nm' dP_nm'),
           dQ_n += tau sum_m dS_nm k_m,  dK_m += tau sum_n dS_nm q_n
  linear:  a_n = phi(q_n),  S_c = sum_{m in C_i} phi(k_m)^T v_m,  z_c = sum_{m in C_i} phi(k_m),
           num_n = a_n S_c,  den_n = a_n . z_c + eps,  O_l[n] = num_n / den_n;
           g_n = dO_l[n] / den_n,  h_n = -(dO_l[n] . num_n) / den_n^2,
           dQ_n += (g_n S_c^T + h_n z_c) (.) phi'(q_n),
           dS_c(i) = sum_{n in R_i} a_n^T g_n,  dz_c(i) = sum_{n in R_i} h_n a_n,
           and every key token m of C_i receives dV_m += phi(k_m) dS_c(i),
           dK_m += (dS_c(i) v_m^T + dz_c(i)) (.) phi'(k_m).
The last line is summed per key block j over the query blocks that did NOT select j
(G_j = sum_{i: j not in sel(i)} dS_c(i)), the transpose of the forward's complement.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from .sla_oracle import (EPS, block_slice, block_summaries, n_blocks, relu, selection_mask,
                         sparse_rows, linear_complement, mix, route_head, _head)


def forward_at(q, k, v, alpha_h, idx, block):
    """The SLA2 forward of one (b, h) at the given selection idx [Nbq, k] (the pieces of
    ``sla_oracle``): returns (O, O_s, O_l)."""
    nq, d = q.shape
    nbk = n_blocks(k.shape[0], block)
    S, z = block_summaries(k, v, block)
    M = selection_mask(idx, nbk)
    o_s = np.zeros((nq, d))
    o_l = np.zeros((nq, d))
    for i in range(n_blocks(nq, block)):
        rows = block_slice(i, nq, block)
        o_s[rows] = sparse_rows(q[rows], k, v, idx[i], block)
        o_l[rows] = linear_complement(q[rows], S, z, M[i])
    return mix(alpha_h, o_s, o_l), o_s, o_l


def _query_block(q, k, v, alpha_h, toks, comp, S, z, rows, dO, tau):
    """The terms of one query block with rows `rows`, the tokens `toks` of its selected key
    blocks and complement indicator `comp` (1 for the key blocks it did not select): its dQ
    rows, its sparse branch's dK, dV contributions on those tokens (toks, dk_t, dv_t),
    dS_c(i), dz_c(i) and its dalpha part."""
    d = k.shape[1]
    dq = np.zeros((len(rows), d))
    o_s = np.zeros((len(rows), d))
    dk_t = dv_t = np.zeros((0, d))
    if len(toks):
        lg = tau * (q[rows] @ k[toks].T)
        p = np.exp(lg - lg.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        o_s = p @ v[toks]
        dos = alpha_h[None, :] * dO
        dv_t = p.T @ dos
        dp = dos @ v[toks].T
        ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        dq += tau * (ds @ k[toks])
        dk_t = tau * (ds.T @ q[rows])
    # linear branch over the complement
    S_c = np.tensordot(comp, S, axes=(0, 0))
    z_c = comp @ z
    a = relu(q[rows])
    num = a @ S_c
    den = a @ z_c + EPS
    o_l = num / den[:, None]
    dol = (1.0 - alpha_h)[None, :] * dO
    g = dol / den[:, None]
    hh = -(dol * num).sum(axis=1) / den ** 2
    dq += (g @ S_c.T + hh[:, None] * z_c[None, :]) * (q[rows] > 0)
    dalpha = (dO * (o_s - o_l)).sum(axis=0)
    return dq, toks, dk_t, dv_t, a.T @ g, a.T @ hh, dalpha


def _tokens(blocks, n, block):
    if len(blocks) == 0:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate([np.arange(n)[block_slice(j, n, block)] for j in blocks])


def backward_head(q, k, v, alpha_h, idx, block, dout):
    """Gradients (dq, dk, dv, dalpha) of sum(dout * O) for one (b, h) at selection idx."""
    nq, d = q.shape
    nkv = k.shape[0]
    nbq, nbk = n_blocks(nq, block), n_blocks(nkv, block)
    tau = 1.0 / math.sqrt(d)
    S, z = block_summaries(k, v, block)
    M = selection_mask(idx, nbk)
    dq = np.zeros((nq, d))
    dk = np.zeros((nkv, d))
    dv = np.zeros((nkv, d))
    dalpha = np.zeros(d)
    dSc = np.zeros((nbq, d, d))
    dzc = np.zeros((nbq, d))
    for i in range(nbq):
        rows = np.arange(nq)[block_slice(i, nq, block)]
        toks = _tokens(idx[i], nkv, block)
        dq_i, toks, dk_t, dv_t, dSc[i], dzc[i], da = _query_block(
            q, k, v, alpha_h, toks, 1.0 - M[i], S, z, rows, dout[rows], tau)
        dq[rows] += dq_i
        dk[toks] += dk_t
        dv[toks] += dv_t
        dalpha += da
    # each key block collects the linear gradients of the query blocks that did not select it
    compT = (1.0 - M).T                               # [Nbk, Nbq]
    G = np.tensordot(compT, dSc, axes=(1, 0))         # [Nbk, d, d]
    gz = compT @ dzc                                  # [Nbk, d]
    for j in range(nbk):
        toks = np.arange(nkv)[block_slice(j, nkv, block)]
        fk = relu(k[toks])
        dv[toks] += fk @ G[j]
        dk[toks] += (v[toks] @ G[j].T + gz[j][None, :]) * (k[toks] > 0)
    return dq, dk, dv, dalpha


def dq_blocks(q, k, v, alpha_h, idx, block, dout, blocks):
    """dQ rows of the listed query blocks only (one (b, h)): the query block's own terms of
    backward_head (its rows' dQ depends on nothing else), for checks at sizes where the
    full backward would be too slow. Returns {i: dq rows of block i}."""
    nq, d = q.shape
    nkv = k.shape[0]
    tau = 1.0 / math.sqrt(d)
    S, z = block_summaries(k, v, block)
    M = selection_mask(idx, n_blocks(nkv, block))
    out = {}
    for i in blocks:
        rows = np.arange(nq)[block_slice(i, nq, block)]
        toks = _tokens(idx[i], nkv, block)
        out[i] = _query_block(q, k, v, alpha_h, toks, 1.0 - M[i], S, z, rows, dout[rows],
                              tau)[0]
    return out


def backward(inputs, dout: np.ndarray, idx: Optional[np.ndarray] = None):
    """Gradients for every (b, h): (dq, dk, dv) float64 shaped like Q, K, V and dalpha
    [H, d] (summed over the batch). dout: [B, H, Nq, d]. idx: the selection (default: the
    learnable router's)."""
    p = inputs.problem
    al = inputs.alpha.astype(np.float64)
    pq = inputs.proj_q.astype(np.float64)
    pk = inputs.proj_k.astype(np.float64)
    dq = np.zeros((p.batch, p.heads, p.n_q, p.head_dim))
    dk = np.zeros((p.batch, p.heads, p.n_kv, p.head_dim))
    dv = np.zeros_like(dk)
    dal = np.zeros((p.heads, p.head_dim))
    for b in range(p.batch):
        for h in range(p.heads):
            q, k, v = _head(inputs, "q", b, h), _head(inputs, "k", b, h), _head(inputs, "v", b, h)
            sel = idx[b, h] if idx is not None else route_head(q, k, pq, pk, p.block, p.top_k).idx
            g = backward_head(q, k, v, al[h], sel, p.block, dout[b, h].astype(np.float64))
            dq[b, h], dk[b, h], dv[b, h] = g[0], g[1], g[2]
            dal[h] += g[3]
    return dq, dk, dv, dal
