"""GPU parity of the training-free (second-order Taylor) router and the forward that uses it.

Selections must match the oracle bit for bit (ties to the lowest index); outputs within
2e-2 x RMS of the oracle forward with the same router.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle                                   # noqa: E402
from oracle import sla_oracle as so             # noqa: E402
from workloads import make_custom, make_inputs, Inputs, bf16_round_bits  # noqa: E402
from tests.gpu_helpers import to_device, check_masks, max_err_over_rms  # noqa: E402

TOL = 2e-2


@pytest.fixture(scope="module")
def sla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_linear_hybrid_amd as s
    return s


CASES = [
    # B, H, nq, nkv, d, top_k, dtype, kind
    (1, 2, 256, 320, 128, 3, "bf16", "smooth"),
    (2, 1, 200, 520, 64, 4, "bf16", "normal"),       # ragged both, d = 64
    (1, 3, 192, 192, 64, 2, "f32", "normal"),
    (1, 2, 640, 1000, 128, 5, "bf16", "smooth"),     # more than 8 query blocks: tiled scores
]


@pytest.mark.parametrize("B,H,nq,nkv,d,top_k,dtype,kind", CASES)
def test_route_taylor_small(sla, B, H, nq, nkv, d, top_k, dtype, kind):
    x = make_custom(B, H, nq, nkv, d, top_k, dtype=dtype, kind=kind, seed=3 * nq + d)
    q, k, v, pq, pk, al = to_device(x)
    idx = sla.sla_route_taylor(q, k, top_k)
    torch.cuda.synchronize()
    check_masks(idx.cpu().numpy(), so.route_full(x, router="taylor"), top_k)


@pytest.mark.parametrize("B,H,nq,nkv,d,top_k,dtype,kind", CASES)
def test_forward_taylor_small(sla, B, H, nq, nkv, d, top_k, dtype, kind):
    x = make_custom(B, H, nq, nkv, d, top_k, dtype=dtype, kind=kind, seed=3 * nq + d)
    q, k, v, pq, pk, al = to_device(x)
    out, idx = sla.sla_forward_taylor(q, k, v, al, top_k)
    torch.cuda.synchronize()
    ref, _ = oracle.forward(x, router="taylor")
    check_masks(idx.cpu().numpy(), so.route_full(x, router="taylor"), top_k)
    err, _ = max_err_over_rms(out.cpu().numpy(), ref)
    print(f"taylor case B={B} H={H} nq={nq} nkv={nkv} d={d} k={top_k}: max-abs/rms {err:.3e}")
    assert err <= TOL


def test_spread_decides_between_equal_means(sla):
    """All key blocks share one mean; the odd ones spread their tokens (+-8 u, alternating)
    along u, the direction the queries lean towards, so they carry more attention mass and
    the 8 of them must be the ones kept."""
    d, nkv, nq = 128, 16 * 64, 128
    x = make_custom(1, 1, nq, nkv, d, 8, dtype="bf16", kind="normal", seed=61)
    rng = np.random.default_rng(5)
    w = rng.standard_normal(d)
    u = w / np.linalg.norm(w)
    q = rng.standard_normal((nq, d)) + w[None]
    base = rng.standard_normal(d) * 0.3
    k = np.tile(base, (nkv, 1))
    sign = np.where(np.arange(64) % 2 == 0, 1.0, -1.0)[:, None]
    for j in range(1, 16, 2):
        k[j * 64:(j + 1) * 64] += 8.0 * sign * u[None]
    qb = bf16_round_bits(q.astype(np.float32))[None, None]
    kb = bf16_round_bits(k.astype(np.float32))[None, None]
    y = Inputs(x.problem, qb, kb, x.v, x.proj_q, x.proj_k, x.alpha, dict(x.meta))
    tq, tk, tv, pq, pk, al = to_device(y)
    idx = sla.sla_route_taylor(tq, tk, 8).cpu().numpy()[0, 0]
    check_masks(idx[None, None], so.route_full(y, router="taylor"), 8)
    assert np.all(idx % 2 == 1)


@pytest.mark.slow
def test_video95_taylor_full(sla):
    x = make_inputs("video95")
    p = x.problem
    q, k, v, pq, pk, al = to_device(x)
    out, idx = sla.sla_forward_taylor(q, k, v, al, p.top_k)
    torch.cuda.synchronize()
    rows, near = check_masks(idx.cpu().numpy(), so.route_full(x, router="taylor"), p.top_k)
    o = out.cpu().numpy()
    refs, gots = [], []
    rng = np.random.default_rng(0)
    for h in (0, 7):
        blocks = rng.choice(p.nbq, size=2, replace=False)
        rws = np.concatenate([np.arange(i * 64, i * 64 + 64) for i in blocks])
        ref, _ = oracle.forward(x, heads=[(0, h)], rows=rws, router="taylor")
        refs.append(ref[0, h, rws])
        gots.append(o[0, h, rws])
    err, rms = max_err_over_rms(np.concatenate(gots), np.concatenate(refs))
    print(f"video95 taylor: rows={rows} near_tie={near} max-abs/rms={err:.3e}")
    assert err <= TOL


def test_profiled_taylor_matches_plain(sla):
    """The stage-timed Taylor forward enqueues the same work as sla_forward_taylor."""
    import ctypes
    x = make_custom(1, 2, 640, 1000, 128, 5, dtype="bf16", kind="smooth", seed=71)
    q, k, v, pq, pk, al = to_device(x)
    out, _ = sla.sla_forward_taylor(q, k, v, al, 5)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(sla.STAGES))]
    for e in evs:
        e.record()                      # torch creates the HIP event on its first record
    torch.cuda.synchronize()
    handles = (ctypes.c_void_p * len(evs))(*[e.cuda_event for e in evs])
    out2 = sla.sla_forward_profiled(q, k, v, None, None, al, 5, handles, taylor=True)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    assert all(evs[2 * i].elapsed_time(evs[2 * i + 1]) >= 0 for i in range(len(sla.STAGES)))
