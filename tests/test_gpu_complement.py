"""GPU parity of the linear complement (SPLA page, section 2.2: the linear term over the
unselected key blocks), region by region: the S_c^T and z_c workspace regions of every query
block against the oracle's direct sum over the unselected blocks, and the whole forward.

The shapes cover the complement's own edges: a ragged second tile of 256 query blocks, ragged
32-block key steps, more than one 960-block bitmap window, steps that every query block of a
tile routed whole (skipped), d = 64 and 128, top-k = 0 (S_c is the total) and top-k = all key
blocks (S_c exactly zero).

Bounds for S_c: every stored S_j and the stored S_c are bf16, rounded to nearest with 8
significant bits (relative error at most 2^-8 each), so |gpu - ref| <= 2^-7 sum_unselected
|S_j| plus fp32 summation error, taken as 1e-5 sum_all |S_j|; z_c is fp32 from fp32 z_j:
1e-5 sum_all z_j while at most half the key blocks are selected (z_tot minus the selected),
else 1e-5 z_c itself (the unselected z_j are summed directly, so a selection of all but one
block must leave that block's z to fp32 accuracy, not z_tot's).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle                                   # noqa: E402
from oracle import sla_oracle as so             # noqa: E402
from workloads import make_custom               # noqa: E402
from tests.gpu_helpers import to_device, check_masks, max_err_over_rms  # noqa: E402

TOL = 2e-2


@pytest.fixture(scope="module")
def sla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_linear_hybrid_amd as s
    return s


CASES = [
    # B, H, nq, nkv, d, top_k, kind
    (1, 2, 64 * 80 - 9, 64 * 40 + 17, 128, 2, "smooth"),    # ragged both; ragged last step
    (1, 1, 64 * 300 + 5, 64 * 70, 64, 6, "normal"),         # two query tiles, d = 64
    (1, 1, 60, 64 * 40, 128, 36, "smooth"),                 # one query block, whole steps routed
    (1, 2, 64 * 30 + 5, 64 * 1200, 64, 40, "smooth"),       # two bitmap windows
    (1, 1, 64 * 40, 64 * 300, 128, 0, "smooth"),            # nothing routed: S_c = total
    (1, 1, 64 * 20, 64 * 12, 128, 12, "normal"),            # everything routed: S_c = 0
    (1, 2, 64 * 64, 64 * 200, 128, 12, "smooth"),           # many query blocks, 6% routed
    (1, 1, 64 * 10, 64 * 40 + 3, 128, 40, "smooth"),        # all but one block routed
    (1, 2, 64 * 8 + 1, 64 * 30, 64, 20, "normal"),          # two thirds routed
]


def oracle_complement(x, b, h):
    """S_c [nbq, d, d] and z_c [nbq, d] straight from the unselected blocks (float64), and
    the bounds' scales sum_unsel |S_j|, sum_all |S_j|, sum_all z_j."""
    p = x.problem
    kk, vv = x.as_f64("k")[b, h], x.as_f64("v")[b, h]
    S, z = so.block_summaries(kk, vv, p.block)
    r = so.route_full(x)[b][h]
    comp = 1.0 - so.selection_mask(r.idx, p.nbk)            # [nbq, nbk]
    Sf = S.reshape(p.nbk, -1)
    sc = (comp @ Sf).reshape(p.nbq, p.head_dim, p.head_dim)
    zc = comp @ z
    scale_un = (comp @ np.abs(Sf)).reshape(sc.shape)
    return sc, zc, scale_un, np.abs(Sf).sum(0).reshape(p.head_dim, p.head_dim), z.sum(0)


@pytest.mark.parametrize("B,H,nq,nkv,d,top_k,kind", CASES)
def test_complement_regions_and_forward(sla, B, H, nq, nkv, d, top_k, kind):
    x = make_custom(B, H, nq, nkv, d, top_k, dtype="bf16", kind=kind, seed=nq + nkv + top_k)
    p = x.problem
    print(f"complement: H={H} nq={nq} nkv={nkv} d={d} k={top_k} {kind}", flush=True)
    q, k, v, pq, pk, al = to_device(x)
    prob = sla.make_problem(q, k, top_k)
    ws = torch.zeros(sla.workspace_size(prob, sla.VARIANT_FORWARD), dtype=torch.uint8,
                     device="cuda")
    out, idx = sla.sla_forward(q, k, v, pq, pk, al, top_k, workspace=ws)
    torch.cuda.synchronize()
    out, idx = out.float().cpu().numpy(), idx.cpu().numpy()
    raw = ws.cpu().numpy()

    def region(name, dtype):
        off, size = sla.workspace_region(prob, name, sla.VARIANT_FORWARD)
        return raw[off:off + size].view(dtype)
    sc_bits = region("sc", np.uint16).reshape(B * H, p.nbq, d, d)
    sc_gpu = (sc_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    zc_gpu = region("zc", np.float32).reshape(B * H, p.nbq, d).astype(np.float64)

    check_masks(idx, so.route_full(x), top_k)
    for b in range(B):
        for h in range(H):
            if top_k >= p.nbk:      # an empty complement is exactly zero
                assert not np.any(sc_gpu[b * H + h]) and not np.any(zc_gpu[b * H + h])
            sc, zc, un, tot, ztot = oracle_complement(x, b, h)
            got = sc_gpu[b * H + h].transpose(0, 2, 1)          # stored as S_c^T
            bound = 2.0 ** -7 * un + 1e-5 * tot[None] + 1e-30
            excess = np.abs(got - sc) / bound
            assert excess.max() <= 1.0, f"S_c off by {excess.max():.2f}x the bound"
            zb = 1e-5 * (zc if 2 * top_k > p.nbk else ztot[None]) + 1e-30
            assert np.all(np.abs(zc_gpu[b * H + h] - zc) <= zb)

    rows = None
    if p.n_q > 4096:                 # sampled query blocks incl. the ragged last one
        blocks = [0, 1, p.nbq // 2, p.nbq - 1]
        rows = np.concatenate([np.arange(i * 64, min(i * 64 + 64, p.n_q)) for i in blocks])
    ref, _ = oracle.forward(x, rows=rows)
    sel = slice(None) if rows is None else rows
    err, _ = max_err_over_rms(out[:, :, sel], ref[:, :, sel])
    print(f"  forward max-abs/rms {err:.3e}")
    assert err <= TOL
