"""Shared helpers of the GPU parity tests: upload seeded inputs, compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

from workloads import Inputs


def to_device(x: Inputs, device="cuda"):
    """Device tensors (q, k, v, proj_q, proj_k, alpha) holding exactly the stored bits."""
    def t(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return (t(x.q), t(x.k), t(x.v), t(x.proj_q), t(x.proj_k), t(x.alpha))


def check_masks(gpu_idx: np.ndarray, routes, top_k: int):
    """Selected block sets must equal the oracle's exactly; rows the oracle flags as near
    ties (boundary gap < 1e-12 of the row's largest score) only need to be a valid top-k.
    ``routes``: nested [b][h] list of oracle Route objects. Returns (#rows, #near-tie rows)."""
    rows = near = 0
    bad = []
    for b, row in enumerate(routes):
        for h, r in enumerate(row):
            g = gpu_idx[b, h]
            for i in range(r.idx.shape[0]):
                rows += 1
                if np.array_equal(g[i], r.idx[i]):
                    continue
                if r.near_tie[i]:
                    near += 1
                    s = r.scores[i]
                    kth = np.sort(s)[::-1][top_k - 1]
                    ok = (len(set(g[i].tolist())) == top_k and np.all(np.diff(g[i]) > 0)
                          and np.all(s[g[i]] >= kth - 1e-12 * np.abs(s).max()))
                    if ok:
                        continue
                bad.append((b, h, i, g[i][:8].tolist(), r.idx[i][:8].tolist()))
    assert not bad, f"{len(bad)} rows differ, first: {bad[:3]}"
    return rows, near


def max_err_over_rms(gpu: np.ndarray, ref: np.ndarray):
    m = ~np.isnan(ref)
    err = np.abs(gpu[m].astype(np.float64) - ref[m])
    rms = np.sqrt(np.mean(ref[m] ** 2))
    return float(err.max() / rms), float(rms)
