"""GPU parity of the piecewise exact-or-approximate forward (sla_forward_pisa).

Selections must match the oracle bit for bit (same learnable router as sla_forward);
outputs within 2e-2 x RMS of the oracle's piecewise forward; the per-block statistics
(centroids, value sums, H_bar) against the oracle's definitions; and the GPU output must
equal dense attention where the expansion is exact (keys constant inside each block).
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from oracle import pisa as op                   # noqa: E402
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
    (1, 2, 256, 320, 128, 2, "bf16", "smooth"),
    (2, 1, 200, 520, 64, 3, "bf16", "normal"),       # ragged both, d = 64
    (1, 2, 192, 700, 128, 4, "f32", "smooth"),       # fp32 inputs, partial last block
    (1, 2, 640, 4200, 128, 9, "bf16", "smooth"),     # two centroid tiles, partial tile
]


def run(sla, x, out_dtype=torch.float32, workspace=None):
    q, k, v, pq, pk, al = to_device(x)
    out, idx = sla.sla_forward_pisa(q, k, v, pq, pk, x.problem.top_k, out_dtype=out_dtype,
                                    workspace=workspace)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), idx.cpu().numpy()


def oracle_pisa(x, heads=None, rows=None):
    return op.forward(x, heads=heads, rows=rows)


@pytest.mark.parametrize("B,H,nq,nkv,d,top_k,dtype,kind", CASES)
def test_pisa_small(sla, B, H, nq, nkv, d, top_k, dtype, kind):
    x = make_custom(B, H, nq, nkv, d, top_k, dtype=dtype, kind=kind, seed=5 * nq + nkv)
    print(f"pisa case B={B} H={H} nq={nq} nkv={nkv} d={d} k={top_k} {dtype} {kind}", flush=True)
    out, idx = run(sla, x)
    ref, _ = oracle_pisa(x)
    check_masks(idx, so.route_full(x), top_k)
    err, _ = max_err_over_rms(out, ref)
    print(f"  max-abs/rms {err:.3e}")
    assert err <= TOL


def test_pisa_grouped_launch(sla):
    """133 query blocks per head, so neighbouring blocks share a workgroup and the last
    group holds one active block; checked on sampled blocks incl. the last."""
    x = make_custom(1, 12, 64 * 132 + 30, 1500, 128, 5, dtype="bf16", kind="smooth", seed=93)
    p = x.problem
    out, idx = run(sla, x)
    check_masks(idx, so.route_full(x), p.top_k)
    blocks = [0, 67, p.nbq - 1]
    rws = np.concatenate([np.arange(i * 64, min(i * 64 + 64, p.n_q)) for i in blocks])
    refs, gots = [], []
    for hh in (0, 11):
        ref, _ = oracle_pisa(x, heads=[(0, hh)], rows=rws)
        refs.append(ref[0, hh, rws])
        gots.append(out[0, hh, rws])
    err, _ = max_err_over_rms(np.concatenate(gots), np.concatenate(refs))
    print(f"pisa grouped: max-abs/rms {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("top_k", [0, 11])
def test_pisa_degenerate_counts(sla, top_k):
    """top_k = 0 (every block through the tail) and top_k = all 11 blocks (dense attention,
    the tail is empty)."""
    x = make_custom(1, 2, 192, 700, 128, top_k, dtype="bf16", kind="smooth", seed=81)
    out, idx = run(sla, x)
    assert idx.shape[-1] == top_k
    ref, _ = oracle_pisa(x)
    err, _ = max_err_over_rms(out, ref)
    print(f"pisa top_k={top_k}: max-abs/rms {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("top_k", [0, 3])
def test_constant_key_blocks_give_dense_attention(sla, top_k):
    """Keys constant inside each block: the tail is exact, so the GPU output must be dense
    softmax attention whatever the router keeps (including a partial last block)."""
    d, nq, nkv = 128, 256, 64 * 9 + 24
    nb = -(-nkv // 64)
    x = make_custom(1, 1, nq, nkv, d, top_k, dtype="bf16", kind="normal", seed=83)
    rng = np.random.default_rng(9)
    k = np.repeat(rng.standard_normal((nb, d)) * 1.5, 64, axis=0)[:nkv]
    kb = bf16_round_bits(k.astype(np.float32))[None, None]
    y = Inputs(x.problem, x.q, kb, x.v, x.proj_q, x.proj_k, x.alpha, dict(x.meta))
    out, _ = run(sla, y)
    qq, kk, vv = (y.as_f64(n)[0, 0] for n in ("q", "k", "v"))
    z = qq @ kk.T / math.sqrt(d)
    w = np.exp(z - z.max(axis=1, keepdims=True))
    dense = (w / w.sum(axis=1, keepdims=True)) @ vv
    err, _ = max_err_over_rms(out[0, 0], dense)
    print(f"constant keys top_k={top_k}: max-abs/rms vs dense {err:.3e}")
    assert err <= TOL


def test_block_statistics(sla):
    """Centroids (hi + lo), value sums and H_bar^T in the workspace against the oracle's
    block_stats."""
    x = make_custom(1, 2, 128, 1000, 128, 3, dtype="bf16", kind="smooth", seed=87)
    p = sla.make_problem(*to_device(x)[:2], 3)
    ws = torch.zeros(sla.workspace_size(p, sla.VARIANT_PISA), dtype=torch.uint8, device="cuda")
    run(sla, x, workspace=ws)
    raw = ws.cpu().numpy()

    def region(name, dtype):
        off, size = sla.workspace_region(p, name, sla.VARIANT_PISA)
        return raw[off:off + size].view(dtype)
    d, nb = 128, 16
    npad = 64
    hbar = region("hbar", np.uint16)
    hbar = (hbar.astype(np.uint32) << 16).view(np.float32).reshape(2, d, d)
    chi = region("cent_hi", np.uint16).astype(np.uint32) << 16
    clo = region("cent_lo", np.uint16).astype(np.uint32) << 16
    cent = (chi.view(np.float32).astype(np.float64) + clo.view(np.float32)).reshape(2, npad, d)
    vsum = region("vsum", np.float16).astype(np.float64).reshape(2, npad, d)
    for h in range(2):
        kk, vv = x.as_f64("k")[0, h], x.as_f64("v")[0, h]
        k_bar, vs, counts, H = op.block_stats(kk, vv, 64)
        hb = H.mean(axis=0)
        assert np.abs(cent[h, :nb] - k_bar).max() <= 1e-5 * np.abs(k_bar).max()
        assert np.all(np.abs(vsum[h, :nb] - vs) <= 1e-3 * np.abs(vs) + 1e-3)
        assert np.abs(hbar[h].T - hb).max() <= 1e-2 * np.abs(hb).max()


def test_pisa_bf16_output(sla):
    x = make_custom(1, 2, 192, 900, 128, 4, dtype="bf16", kind="normal", seed=89)
    o32, _ = run(sla, x)
    o16, _ = run(sla, x, out_dtype=torch.bfloat16)
    want = torch.from_numpy(o32).bfloat16().float().numpy()
    assert np.abs(o16 - want).max() <= 1e-6 + 1e-2 * np.abs(want).max()


def test_profiled_pisa_matches_plain(sla):
    import ctypes
    x = make_custom(1, 2, 640, 1000, 128, 5, dtype="bf16", kind="smooth", seed=91)
    q, k, v, pq, pk, al = to_device(x)
    out, _ = sla.sla_forward_pisa(q, k, v, pq, pk, 5)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(sla.STAGES))]
    for e in evs:
        e.record()                      # torch creates the HIP event on its first record
    torch.cuda.synchronize()
    handles = (ctypes.c_void_p * len(evs))(*[e.cuda_event for e in evs])
    out2 = sla.sla_forward_profiled(q, k, v, pq, pk, None, 5, handles, pisa=True)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


def sampled_full(sla, name, heads, nblocks):
    x = make_inputs(name)
    p = x.problem
    out, idx = run(sla, x)
    rows, near = check_masks(idx, so.route_full(x), p.top_k)
    rng = np.random.default_rng(1)
    refs, gots = [], []
    for b, h in heads:
        blocks = rng.choice(p.nbq, size=nblocks, replace=False)
        rws = np.concatenate([np.arange(i * 64, min(i * 64 + 64, p.n_q)) for i in blocks])
        ref, _ = oracle_pisa(x, heads=[(b, h)], rows=rws)
        refs.append(ref[b, h, rws])
        gots.append(out[b, h, rws])
    err, rms = max_err_over_rms(np.concatenate(gots), np.concatenate(refs))
    print(f"{name} pisa: rows={rows} near_tie={near} max-abs/rms={err:.3e}")
    return err


@pytest.mark.slow
def test_video95_pisa_full(sla):
    assert sampled_full(sla, "video95", [(0, 0), (0, 7)], 2) <= TOL


@pytest.mark.slow
def test_video90_pisa_full(sla):
    """75600 tokens: a partial last block (16 tokens) in the tail and the exact branch."""
    assert sampled_full(sla, "video90", [(0, 3)], 2) <= TOL
