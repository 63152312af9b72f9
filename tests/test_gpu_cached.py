"""GPU parity of the key/value summary cache and the cached (decode) forward.

The cache contents are checked against the oracle's definitions (projected block means,
the totals of the per-block summaries); incremental updates against a one-shot build; the
cached forward against the oracle forward (masks bit for bit, outputs within 2e-2 x RMS)
and against sla_forward on the same inputs.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle                                   # noqa: E402
from oracle import sla_oracle as so             # noqa: E402
from workloads import make_custom, make_inputs  # noqa: E402
from tests.gpu_helpers import to_device, check_masks, max_err_over_rms  # noqa: E402

TOL = 2e-2


@pytest.fixture(scope="module")
def sla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_linear_hybrid_amd as s
    return s


def cache_views(sla, p, cache):
    """(S_tot^T [BH, d, d] fp32, z_tot [BH, d] fp32, k~ [nbk, BH, d] fp64) of a cache."""
    BH, d = p.batch * p.heads, p.head_dim
    nbk = -(-p.n_kv // 64)
    raw = cache.cpu().numpy()
    ztot_off = -(-(BH * d * d * 4) // 256) * 256
    kt_off = -(-(ztot_off + BH * d * 4) // 256) * 256
    assert sla.kv_cache_size(p) == kt_off + nbk * BH * d * 8
    st = raw[:BH * d * d * 4].view(np.float32).reshape(BH, d, d)
    zt = raw[ztot_off:ztot_off + BH * d * 4].view(np.float32).reshape(BH, d)
    kt = raw[kt_off:kt_off + nbk * BH * d * 8].view(np.float64).reshape(nbk, BH, d)
    return st, zt, kt


def build_cache(sla, k, v, pk, steps):
    """Cache built by successive updates at the token counts in `steps` (last = n_kv)."""
    p = sla.make_problem(k, k, 0)
    cache = torch.zeros(sla.kv_cache_size(p), dtype=torch.uint8, device="cuda")
    done = 0
    for n in steps:
        sla.sla_kv_cache_update(k[:, :, :n].contiguous(), v[:, :, :n].contiguous(), pk, cache,
                                n_done=done)
        done = n
    torch.cuda.synchronize()
    return p, cache


def test_cache_matches_definitions(sla):
    x = make_custom(1, 2, 64, 1000, 128, 4, dtype="bf16", kind="smooth", seed=41)
    q, k, v, pq, pk, al = to_device(x)
    p, cache = build_cache(sla, k, v, pk, [x.problem.n_kv])
    st, zt, kt = cache_views(sla, p, cache)
    for h in range(2):
        kk = x.as_f64("k")[0, h]
        vv = x.as_f64("v")[0, h]
        want_kt = so.project(so.pool_blocks(kk, 64), x.proj_k.astype(np.float64))
        assert np.allclose(kt[:, h], want_kt, rtol=1e-12, atol=1e-12)
        S, z = so.block_summaries(kk, vv, 64)
        s_ref = S.sum(axis=0)                     # [r][c]
        assert np.abs(st[h].T - s_ref).max() <= 1e-5 * np.abs(s_ref).max()
        assert np.abs(zt[h] - z.sum(axis=0)).max() <= 1e-5 * np.abs(z.sum(axis=0)).max()


def test_incremental_updates_match_one_build(sla):
    """Appends that start and end inside blocks give the same cache as one build: k~ bit
    for bit (every touched block is re-pooled from all its tokens), totals up to fp32
    summation order."""
    x = make_custom(2, 1, 64, 1100, 64, 3, dtype="bf16", kind="normal", seed=43)
    q, k, v, pq, pk, al = to_device(x)
    p, one = build_cache(sla, k, v, pk, [1100])
    _, inc = build_cache(sla, k, v, pk, [100, 130, 640, 641, 1100])
    s1, z1, k1 = cache_views(sla, p, one)
    s2, z2, k2 = cache_views(sla, p, inc)
    assert np.array_equal(k1, k2)
    assert np.abs(s1 - s2).max() <= 1e-5 * np.abs(s1).max()
    assert np.abs(z1 - z2).max() <= 1e-5 * np.abs(z1).max()


def run_cached(sla, x, out_dtype=torch.float32):
    q, k, v, pq, pk, al = to_device(x)
    _, cache = build_cache(sla, k, v, pk, [x.problem.n_kv])
    out, idx = sla.sla_forward_cached(q, k, v, pq, al, x.problem.top_k, cache,
                                      out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), idx.cpu().numpy()


CASES = [
    # B, H, nq, nkv, d, top_k, kind
    (2, 2, 64, 1500, 128, 8, "normal"),      # decode chunk, ragged key tail
    (1, 3, 130, 900, 64, 5, "smooth"),       # several query blocks, ragged both
    (1, 2, 64, 4096, 128, 40, "smooth"),     # many selected blocks per part
    (1, 1, 40, 700, 128, 1, "normal"),       # one selected block, partial query block
]


@pytest.mark.parametrize("B,H,nq,nkv,d,top_k,kind", CASES)
def test_cached_forward_small(sla, B, H, nq, nkv, d, top_k, kind):
    x = make_custom(B, H, nq, nkv, d, top_k, dtype="bf16", kind=kind, seed=nkv + d)
    print(f"cached case B={B} H={H} nq={nq} nkv={nkv} d={d} k={top_k} {kind}", flush=True)
    out, idx = run_cached(sla, x)
    ref, _ = oracle.forward(x)
    check_masks(idx, oracle.sla_oracle.route_full(x), top_k)
    err, _ = max_err_over_rms(out, ref)
    print(f"  max-abs/rms {err:.3e}")
    assert err <= TOL, f"max-abs/rms {err:.3e}"


@pytest.mark.parametrize("top_k", [0, 16])
def test_cached_degenerate_counts(sla, top_k):
    """top_k = 0 (linear branch alone) and top_k = all 16 key blocks (empty complement)."""
    x = make_custom(1, 2, 64, 1024, 128, top_k, dtype="bf16", kind="normal", seed=47)
    out, idx = run_cached(sla, x)
    ref, _ = oracle.forward(x)
    assert idx.shape[-1] == top_k
    err, _ = max_err_over_rms(out, ref)
    assert err <= TOL


def test_cached_matches_plain_forward(sla):
    x = make_custom(1, 2, 192, 2000, 128, 6, dtype="bf16", kind="smooth", seed=53)
    out_c, idx_c = run_cached(sla, x)
    q, k, v, pq, pk, al = to_device(x)
    out_f, idx_f = sla.sla_forward(q, k, v, pq, pk, al, 6)
    torch.cuda.synchronize()
    assert np.array_equal(idx_c, idx_f.cpu().numpy())
    err, _ = max_err_over_rms(out_c, out_f.cpu().numpy())
    assert err <= 1e-2


def test_cached_bf16_output(sla):
    x = make_custom(1, 2, 64, 1200, 128, 6, dtype="bf16", kind="normal", seed=59)
    o32, _ = run_cached(sla, x)
    o16, _ = run_cached(sla, x, out_dtype=torch.bfloat16)
    want = torch.from_numpy(o32).bfloat16().float().numpy()
    assert np.abs(o16 - want).max() <= 1e-6 + 1e-2 * np.abs(want).max()


@pytest.mark.slow
def test_longctx_cached_full(sla):
    x = make_inputs("longctx")
    p = x.problem
    out, idx = run_cached(sla, x)
    rows, near = check_masks(idx, oracle.sla_oracle.route_full(x), p.top_k)
    assert near == 0
    refs, gots = [], []
    for b, h in [(0, 0), (1, 7), (3, 31)]:
        ref, _ = oracle.forward(x, heads=[(b, h)])
        refs.append(ref[b, h])
        gots.append(out[b, h])
    err, rms = max_err_over_rms(np.concatenate(gots), np.concatenate(refs))
    print(f"longctx cached: rows={rows} near_tie={near} max-abs/rms={err:.3e} rms={rms:.4f}")
    assert err <= TOL


# ----------------------------------------------------------------------------- cache path
# sla_forward with at most 8 query blocks per head over at least 256 key blocks builds the
# summary cache in its workspace and runs the cached forward.
FEW_CASES = [
    (1, 4, 100, 64 * 300, 128, 10, "smooth"),     # two query blocks, ragged
    (2, 2, 64 * 8, 64 * 256 + 40, 64, 7, "normal"),  # 8 query blocks, partial last key block
    (1, 2, 64, 64 * 300, 128, 0, "smooth"),       # nothing routed: the linear branch alone
    (1, 1, 30, 64 * 260, 128, 260, "normal"),     # everything routed: the complement is empty
]


@pytest.mark.parametrize("B,H,nq,nkv,d,top_k,kind", FEW_CASES)
def test_forward_cache_path(sla, B, H, nq, nkv, d, top_k, kind):
    x = make_custom(B, H, nq, nkv, d, top_k, dtype="bf16", kind=kind, seed=nq + nkv + top_k)
    print(f"cache path B={B} H={H} nq={nq} nkv={nkv} d={d} k={top_k} {kind}", flush=True)
    q, k, v, pq, pk, al = to_device(x)
    out, idx = sla.sla_forward(q, k, v, pq, pk, al, top_k)
    torch.cuda.synchronize()
    out, idx = out.cpu().numpy(), idx.cpu().numpy()
    check_masks(idx, oracle.sla_oracle.route_full(x), top_k)
    ref, _ = oracle.forward(x)
    err, _ = max_err_over_rms(out, ref)
    print(f"  max-abs/rms {err:.3e}")
    assert err <= TOL, f"max-abs/rms {err:.3e}"
    # same selection and the same arithmetic as building the cache and calling the cached
    # forward
    out_c, idx_c = run_cached(sla, x)
    assert np.array_equal(idx, idx_c) and np.array_equal(out, out_c)


def test_forward_cache_path_bf16_output_and_profiled(sla):
    x = make_custom(1, 3, 64 * 2, 64 * 270, 128, 9, dtype="bf16", kind="smooth", seed=77)
    q, k, v, pq, pk, al = to_device(x)
    o32, _ = sla.sla_forward(q, k, v, pq, pk, al, 9)
    o16, _ = sla.sla_forward(q, k, v, pq, pk, al, 9, out_dtype=torch.bfloat16)
    import ctypes
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(sla.STAGES))]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    handles = (ctypes.c_void_p * len(evs))(*[e.cuda_event for e in evs])
    op = sla.sla_forward_profiled(q, k, v, pq, pk, al, 9, handles)
    torch.cuda.synchronize()
    assert torch.equal(op, o32)
    assert torch.equal(o16, o32.bfloat16())
    times = [evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(len(sla.STAGES))]
    assert all(t >= 0 for t in times)
