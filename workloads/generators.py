"""Seeded generators for the five synthetic workloads and for small custom shapes.

Workloads (all seeded with numpy PCG64, a fresh generator per workload, draws in the
order Q, K, V, proj_q, proj_k, alpha, then any structural choices):

* ``tiny``        B=1 H=2 N=1024 d=64 fp32, block 64, top-k 4; Q,K,V ~ N(0,1).
* ``video95``     B=1 H=12 N=32768 (latent grid 8x64x64) d=128 bf16, top-k 26.
* ``video90``     B=1 H=40 N=75600 (grid 21x45x80) d=128 bf16, top-k 118, last block
                  holds 16 tokens.
* ``video95_fp8`` byte-identical inputs to ``video95``; the sparse branch runs in e4m3.
* ``longctx``     B=4 H=32, 64 query tokens against 131072 keys, d=128 bf16, top-k 64,
                  1% of key blocks shifted toward the head's mean query.

Video workloads: Q and K are, per (batch, head, channel), a sum of 16 sinusoids over the
(t, y, x) latent grid with per-axis frequencies uniform in [-0.2, 0.2] rad/token, phases
uniform in [0, 2pi) and N(0,1) amplitudes, plus N(0, 0.5^2) noise; V ~ N(0,1). Token n
sits at grid point (t, y, x) with n = (t*Hg + y)*Wg + x. proj_q, proj_k are d x d with
N(0, 1/d) entries and alpha = sigmoid(N(0,1)) per head and channel.

Nothing here performs pooling, routing, attention or any other step of the method; the
only arithmetic is drawing numbers and rounding them to the storage dtype.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class Problem:
    """Shape and routing parameters of one SLA forward problem."""
    batch: int
    heads: int
    n_q: int
    n_kv: int
    head_dim: int
    block: int
    top_k: int
    dtype: str                 # "bf16" or "f32": storage type of Q, K, V
    name: str = "custom"
    grid: Optional[tuple] = None   # (T, Hg, Wg) latent grid for video workloads

    @property
    def nbq(self) -> int:
        return -(-self.n_q // self.block)

    @property
    def nbk(self) -> int:
        return -(-self.n_kv // self.block)

    @property
    def sparsity(self) -> float:
        return 1.0 - self.top_k / self.nbk


@dataclass
class Inputs:
    """Host copies of one problem's inputs.

    q, k, v: uint16 bf16 bit patterns when ``problem.dtype == "bf16"``, else float32;
    shape [B, H, N, d] row-major. proj_q, proj_k: float32 [d_in, d_out]. alpha: float32
    [H, d].
    """
    problem: Problem
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    proj_q: np.ndarray
    proj_k: np.ndarray
    alpha: np.ndarray
    meta: dict = field(default_factory=dict)

    def as_f64(self, name: str) -> np.ndarray:
        """Exact float64 upcast of a stored tensor."""
        x = getattr(self, name)
        if x.dtype == np.uint16:
            return bf16_bits_to_f32(x).astype(np.float64)
        return x.astype(np.float64)


CONFIGS = {
    "tiny": Problem(1, 2, 1024, 1024, 64, 64, 4, "f32", "tiny"),
    "video95": Problem(1, 12, 32768, 32768, 128, 64, 26, "bf16", "video95", (8, 64, 64)),
    "video90": Problem(1, 40, 75600, 75600, 128, 64, 118, "bf16", "video90", (21, 45, 80)),
    "video95_fp8": Problem(1, 12, 32768, 32768, 128, 64, 26, "bf16", "video95_fp8", (8, 64, 64)),
    "longctx": Problem(4, 32, 64, 131072, 128, 64, 64, "bf16", "longctx"),
}


# --------------------------------------------------------------------------- storage rounding
def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    r = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        r = np.where(nan, ((u >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16), r)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def sha256_of(*arrays: np.ndarray) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


# --------------------------------------------------------------------------- field generators
def _smooth_field(rng: np.random.Generator, grid, d: int, n_sin: int = 16,
                  fmax: float = 0.2, noise: float = 0.5) -> np.ndarray:
    """One (batch, head) of the smooth-field generator: float64 [N, d]."""
    T, Hg, Wg = grid
    freq = rng.uniform(-fmax, fmax, size=(d, n_sin, 3))
    phase = rng.uniform(0.0, 2.0 * np.pi, size=(d, n_sin))
    amp = rng.standard_normal(size=(d, n_sin))
    t = np.arange(T, dtype=np.float64)
    y = np.arange(Hg, dtype=np.float64)
    x = np.arange(Wg, dtype=np.float64)
    # sin(a + b) = sin(a)cos(b) + cos(a)sin(b) with a over (t, y) and b over x, so each
    # channel's field is a product of a [T*Hg, 2S] and a [2S, Wg] matrix.
    a = (freq[:, :, 0, None, None] * t[None, None, :, None]
         + freq[:, :, 1, None, None] * y[None, None, None, :]
         + phase[:, :, None, None]).reshape(d, n_sin, T * Hg)          # [d, S, TY]
    b = freq[:, :, 2, None] * x[None, None, :]                            # [d, S, Wg]
    left = np.concatenate([amp[:, :, None] * np.sin(a), amp[:, :, None] * np.cos(a)], axis=1)
    right = np.concatenate([np.cos(b), np.sin(b)], axis=1)               # [d, 2S, Wg]
    field_ = np.matmul(left.transpose(0, 2, 1), right)                    # [d, TY, Wg]
    out = field_.reshape(d, T * Hg * Wg).T.copy()                         # [N, d]
    out += noise * rng.standard_normal(size=out.shape)
    return out


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    return bf16_round_bits(x32) if dtype == "bf16" else x32


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _proj(rng, d):
    return (rng.standard_normal(size=(d, d)) / np.sqrt(d)).astype(np.float32)


def _alpha(rng, h, d):
    return _sigmoid(rng.standard_normal(size=(h, d))).astype(np.float32)


def _normal_tensor(rng, shape, dtype):
    """N(0,1) tensor drawn per (batch, head) in C order, rounded to the storage dtype."""
    B, H, N, d = shape
    out = np.empty(shape, dtype=np.uint16 if dtype == "bf16" else np.float32)
    for b in range(B):
        for h in range(H):
            out[b, h] = _store(rng.standard_normal(size=(N, d)), dtype)
    return out


def make_inputs(name: str, seed: int = 0, heads: Optional[int] = None) -> Inputs:
    """Inputs of a named workload. ``heads`` truncates H (draws for the kept heads are
    identical to the full workload's, because each tensor is drawn head by head and the
    later tensors are re-seeded per tensor)."""
    p = CONFIGS[name]
    if heads is not None:
        p = Problem(p.batch, heads, p.n_q, p.n_kv, p.head_dim, p.block, p.top_k, p.dtype,
                    p.name, p.grid)
    ss = np.random.SeedSequence(seed)
    # One child stream per tensor so that truncating heads keeps the kept heads identical.
    streams = [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(7)]
    B, H, d = p.batch, p.heads, p.head_dim
    meta = {"workload": p.name, "seed": seed}
    if p.grid is not None:
        qs, ks = [], []
        q = np.empty((B, H, p.n_q, d), np.uint16)
        k = np.empty((B, H, p.n_kv, d), np.uint16)
        full = p.grid[0] * p.grid[1] * p.grid[2]
        for b in range(B):
            for h in range(H):
                q[b, h] = _store(_smooth_field(streams[0], p.grid, d)[: p.n_q], "bf16")
        for b in range(B):
            for h in range(H):
                k[b, h] = _store(_smooth_field(streams[1], p.grid, d)[: p.n_kv], "bf16")
        assert full == p.n_q == p.n_kv
        v = _normal_tensor(streams[2], (B, H, p.n_kv, d), "bf16")
        pq = _proj(streams[3], d)
        pk = _proj(streams[4], d)
        al = _alpha(streams[5], H, d)
    elif name == "longctx":
        q = _normal_tensor(streams[0], (B, H, p.n_q, d), "bf16")
        k = _normal_tensor(streams[1], (B, H, p.n_kv, d), "bf16")
        v = _normal_tensor(streams[2], (B, H, p.n_kv, d), "bf16")
        pq = np.eye(d, dtype=np.float32)
        pk = np.eye(d, dtype=np.float32)
        al = _alpha(streams[5], H, d)
        # 1% of key blocks per (b, h) shifted by +2 along the unit mean-query direction.
        n_sal = int(0.01 * p.nbk)
        salient = np.empty((B, H, n_sal), np.int64)
        for b in range(B):
            for h in range(H):
                blocks = np.sort(streams[6].choice(p.nbk, size=n_sal, replace=False))
                salient[b, h] = blocks
                qm = bf16_bits_to_f32(q[b, h]).astype(np.float64).mean(axis=0)
                u = qm / np.linalg.norm(qm)
                kk = bf16_bits_to_f32(k[b, h]).astype(np.float64)
                for j in blocks:
                    kk[j * p.block:(j + 1) * p.block] += 2.0 * u
                    k[b, h, j * p.block:(j + 1) * p.block] = _store(
                        kk[j * p.block:(j + 1) * p.block], "bf16")
        meta["salient_blocks"] = salient
    else:  # tiny
        q = _normal_tensor(streams[0], (B, H, p.n_q, d), p.dtype)
        k = _normal_tensor(streams[1], (B, H, p.n_kv, d), p.dtype)
        v = _normal_tensor(streams[2], (B, H, p.n_kv, d), p.dtype)
        pq = _proj(streams[3], d)
        pk = _proj(streams[4], d)
        al = _alpha(streams[5], H, d)
    return Inputs(p, q, k, v, pq, pk, al, meta)


def make_custom(batch: int, heads: int, n_q: int, n_kv: int, head_dim: int, top_k: int,
                dtype: str = "bf16", seed: int = 0, kind: str = "normal",
                block: int = 64, scale: float = 1.0) -> Inputs:
    """Small seeded problems for parity tests.

    kind: "normal" (Q, K, V ~ N(0, scale^2)) or "smooth" (a 1-D smooth field along the
    token axis plus noise, which gives spatially coherent routing like the video inputs).
    """
    p = Problem(batch, heads, n_q, n_kv, head_dim, block, top_k, dtype, f"custom_{kind}")
    rng = np.random.Generator(np.random.PCG64(seed))
    B, H, d = batch, heads, head_dim

    def tensor(n):
        out = np.empty((B, H, n, d), dtype=np.uint16 if dtype == "bf16" else np.float32)
        for b in range(B):
            for h in range(H):
                if kind == "smooth":
                    f = rng.uniform(-0.05, 0.05, size=(d, 8))
                    ph = rng.uniform(0, 2 * np.pi, size=(d, 8))
                    a = rng.standard_normal(size=(d, 8))
                    t = np.arange(n, dtype=np.float64)
                    x = (a[None] * np.sin(t[:, None, None] * f[None] + ph[None])).sum(-1)
                    x += 0.5 * rng.standard_normal(size=(n, d))
                else:
                    x = rng.standard_normal(size=(n, d))
                out[b, h] = _store(scale * x, dtype)
        return out

    q = tensor(n_q)
    k = tensor(n_kv)
    v = np.empty((B, H, n_kv, d), dtype=np.uint16 if dtype == "bf16" else np.float32)
    for b in range(B):
        for h in range(H):
            v[b, h] = _store(rng.standard_normal(size=(n_kv, d)), dtype)
    pq = _proj(rng, d)
    pk = _proj(rng, d)
    al = _alpha(rng, H, d)
    return Inputs(p, q, k, v, pq, pk, al, {"workload": p.name, "seed": seed})
