"""GPU parity of the backward (sla_backward) against the float64 gradient oracle.

The selection is the forward's (checked bit for bit against the oracle's router first); the
oracle then differentiates the forward at that selection. Each gradient must satisfy
max-abs error <= tolerance x RMS of the oracle's gradient.

Exact branch: the GPU recomputes P in f16 from the row log-sum-exp, carries dO_s in f16 and
dS as bf16 high + low parts, fp32 accumulation; dV = P^T dO_s sums up to 64 x top-k rounded
products per entry, so its error is a few f16 roundings (2^-11) of the largest terms times
the square root of the number of terms: TOL = 3e-2 of the RMS.
Linear branch: S_j, S_c, g, dS_c and G are carried as bf16 high + low parts (16 significant
bits) and summed in fp32, so the branch is close to fp32 even though its gradients are
differences of nearly equal terms (the covariance of phi(k) and v over the complement):
TOL_LINEAR = 1e-3 where it is the only branch (top-k = 0, or alpha = 0 for dQ, dK, dV).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle                                   # noqa: E402
from oracle import backward as bw               # noqa: E402
from workloads import make_custom               # noqa: E402
from tests.gpu_helpers import to_device, check_masks  # noqa: E402

TOL = 3e-2
TOL_LINEAR = 1e-3


@pytest.fixture(scope="module")
def sla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_linear_hybrid_amd as s
    return s


def rel_err(got, ref):
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return float(np.abs(got.astype(np.float64) - ref).max() / max(rms, 1e-30)), rms


CASES = [
    # B, H, nq, nkv, d, top_k, kind, dout dtype
    (1, 2, 256, 256, 128, 2, "smooth", "f32"),
    (1, 2, 300, 700, 128, 3, "smooth", "f32"),      # ragged both, n_q != n_kv
    (2, 1, 200, 520, 64, 4, "normal", "f32"),       # d = 64
    (1, 2, 130, 400, 128, 0, "normal", "f32"),      # nothing routed: linear branch alone
    (1, 1, 190, 300, 128, 5, "smooth", "f32"),      # every block routed: no linear branch
    (1, 2, 320, 448, 128, 3, "smooth", "bf16"),     # bf16 upstream gradient
    # at most 8 query blocks per head (all the cases above): the key kernel sums each G_j
    # from the dS_c(i) itself; more: G_j from the transposed complement
    (1, 2, 128, 64 * 40 - 9, 128, 3, "normal", "f32"),  # 2 query blocks over 40 key blocks
    (1, 2, 670, 700, 128, 3, "smooth", "f32"),      # 11 query blocks, ragged
    (1, 1, 64 * 9, 64 * 12, 64, 4, "normal", "f32"),  # 9 query blocks, d = 64
]


@pytest.mark.parametrize("B,H,nq,nkv,d,top_k,kind,gdt", CASES)
def test_backward_matches_oracle(sla, B, H, nq, nkv, d, top_k, kind, gdt):
    print(f"backward case B={B} H={H} nq={nq} nkv={nkv} d={d} k={top_k} {kind} dout={gdt}",
          flush=True)
    x = make_custom(B, H, nq, nkv, d, top_k, dtype="bf16", kind=kind, seed=nq + nkv + d + top_k)
    q, k, v, pq, pk, al = to_device(x)
    out_dtype = torch.float32 if gdt == "f32" else torch.bfloat16
    _, idx = sla.sla_forward(q, k, v, pq, pk, al, top_k, out_dtype=out_dtype)
    check_masks(idx.cpu().numpy(), oracle.sla_oracle.route_full(x), top_k)
    rng = np.random.default_rng(nq + 7)
    dout = rng.standard_normal((B, H, nq, d)).astype(np.float32)
    dout_t = torch.from_numpy(dout).cuda().to(out_dtype)
    dout64 = dout_t.float().cpu().numpy().astype(np.float64)
    dq, dk, dv, dal = sla.sla_backward(q, k, v, al, dout_t, idx)
    torch.cuda.synchronize()
    rq, rk, rv, ral = bw.backward(x, dout64, idx=idx.cpu().numpy())
    errs = {}
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv), ("dalpha", dal, ral)):
        errs[name] = rel_err(got.cpu().numpy(), ref)
    print("  " + ", ".join(f"{n} {e:.2e} (rms {r:.3g})" for n, (e, r) in errs.items()), flush=True)
    tol = TOL_LINEAR if top_k == 0 else TOL
    for name, (e, _) in errs.items():
        assert e <= tol, f"{name}: max-abs/rms {e:.3e}"


def test_backward_is_bit_reproducible(sla):
    x = make_custom(1, 2, 300, 700, 128, 3, dtype="bf16", kind="smooth", seed=5)
    q, k, v, pq, pk, al = to_device(x)
    _, idx = sla.sla_forward(q, k, v, pq, pk, al, 3)
    dout = torch.randn(q.shape, device="cuda", generator=torch.Generator("cuda").manual_seed(3))
    first = sla.sla_backward(q, k, v, al, dout, idx)
    second = sla.sla_backward(q, k, v, al, dout, idx)
    torch.cuda.synchronize()
    for a_, b_ in zip(first, second):
        assert torch.equal(a_, b_)


@pytest.mark.parametrize("alpha_value", [1.0, 0.0])
def test_backward_single_branch(sla, alpha_value):
    """alpha = 1 leaves only the exact branch's gradients, alpha = 0 only the linear branch's
    (and dalpha); each against the oracle on its own."""
    x = make_custom(1, 2, 300, 700, 128, 3, dtype="bf16", kind="smooth", seed=33)
    x.alpha[:] = alpha_value
    q, k, v, pq, pk, al = to_device(x)
    _, idx = sla.sla_forward(q, k, v, pq, pk, al, 3)
    check_masks(idx.cpu().numpy(), oracle.sla_oracle.route_full(x), 3)
    dout = np.random.default_rng(9).standard_normal(q.shape).astype(np.float32)
    dq, dk, dv, dal = sla.sla_backward(q, k, v, al, torch.from_numpy(dout).cuda(), idx)
    torch.cuda.synchronize()
    rq, rk, rv, ral = bw.backward(x, dout.astype(np.float64), idx=idx.cpu().numpy())
    errs = {n: rel_err(g.cpu().numpy(), r) for n, g, r in
            (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv), ("dalpha", dal, ral))}
    print(f"alpha = {alpha_value}: " + ", ".join(f"{n} {e:.2e}" for n, (e, _) in errs.items()),
          flush=True)
    for name, (e, _) in errs.items():
        tol = TOL_LINEAR if alpha_value == 0.0 and name != "dalpha" else TOL
        assert e <= tol, f"{name}: max-abs/rms {e:.3e}"


@pytest.mark.slow
def test_backward_video95_sampled_dq(sla):
    """Full video95 shape (B=1, H=12, 32768 tokens, d=128, top-k 26): the GPU's dQ on
    sampled query blocks of two heads against the oracle's per-block dQ (which depends only
    on the block's own rows, selection and complement)."""
    from workloads import make_inputs
    x = make_inputs("video95")
    q, k, v, pq, pk, al = to_device(x)
    _, idx = sla.sla_forward(q, k, v, pq, pk, al, x.problem.top_k)
    rng = np.random.default_rng(95)
    dout = rng.standard_normal(q.shape).astype(np.float32)
    dq, _, _, _ = sla.sla_backward(q, k, v, al, torch.from_numpy(dout).cuda(), idx)
    torch.cuda.synchronize()
    dq = dq.cpu().numpy()
    idx = idx.cpu().numpy()
    got, want = [], []
    for h in (0, 7):
        blocks = sorted(rng.choice(x.problem.nbq, size=3, replace=False).tolist())
        ref = bw.dq_blocks(x.as_f64("q")[0, h], x.as_f64("k")[0, h], x.as_f64("v")[0, h],
                           x.alpha[h].astype(np.float64), idx[0, h], 64,
                           dout[0, h].astype(np.float64), blocks)
        for i in blocks:
            got.append(dq[0, h, 64 * i:64 * i + 64])
            want.append(ref[i])
    err, rms = rel_err(np.concatenate(got), np.concatenate(want))
    print(f"video95 backward, sampled dq: max-abs/rms {err:.2e} (rms {rms:.3g})", flush=True)
    assert err <= TOL


@pytest.mark.slow
def test_backward_longctx_sampled_heads(sla):
    """Full longctx shape (B=4, H=32, 64 queries over 131072 keys, d=128, top-k 64: one query
    block per head, so the few-query-block path with its linear-only key kernel): every
    gradient of head 5 in all four batches (hence dalpha[5] too) and of (b=2, h=20), all
    131072 keys of each, against the oracle's per-head backward at the GPU's selection.
    dK and dV hold two populations: the 4096 keys of the routed blocks carry the exact
    branch's gradients, the other 126976 only the linear branch's, orders of magnitude
    smaller. Each is held to its own RMS: TOL for the routed keys, TOL_LINEAR for the others
    (the linear branch alone, as with top-k = 0)."""
    from workloads import make_inputs, bf16_bits_to_f32
    x = make_inputs("longctx")
    p = x.problem
    q, k, v, pq, pk, al = to_device(x)
    _, idx = sla.sla_forward(q, k, v, pq, pk, al, p.top_k)
    rng = np.random.default_rng(131)
    dout = rng.standard_normal(q.shape).astype(np.float32)
    dq, dk, dv, dal = sla.sla_backward(q, k, v, al, torch.from_numpy(dout).cuda(), idx)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    f64 = lambda a, b, h: bf16_bits_to_f32(a[b, h]).astype(np.float64)   # noqa: E731
    ral = np.zeros(p.head_dim)
    worst = {}
    for b, h in ((0, 5), (1, 5), (2, 5), (3, 5), (2, 20)):
        rq, rk, rv, ra = bw.backward_head(f64(x.q, b, h), f64(x.k, b, h), f64(x.v, b, h),
                                          x.alpha[h].astype(np.float64), idx[b, h], p.block,
                                          dout[b, h].astype(np.float64))
        if h == 5:
            ral += ra
        routed = np.zeros(p.n_kv, dtype=bool)
        for j in np.unique(idx[b, h]):
            routed[p.block * j:p.block * (j + 1)] = True
        checks = [("dq", dq[b, h].cpu().numpy(), rq)]
        for name, got, ref in (("dk", dk[b, h], rk), ("dv", dv[b, h], rv)):
            g = got.cpu().numpy()
            checks += [(name + " routed", g[routed], ref[routed]),
                       (name + " linear-only", g[~routed], ref[~routed])]
        for name, got, ref in checks:
            e, rms = rel_err(got, ref)
            if e > worst.get(name, (0.0, 0.0))[0]:
                worst[name] = (e, rms)
    worst["dalpha"] = rel_err(dal[5].cpu().numpy(), ral)
    print("longctx backward, sampled heads: " +
          ", ".join(f"{n} {e:.2e} (rms {r:.3g})" for n, (e, r) in worst.items()), flush=True)
    for name, (e, _) in worst.items():
        tol = TOL_LINEAR if name.endswith("linear-only") else TOL
        assert e <= tol, f"{name}: max-abs/rms {e:.3e}"
