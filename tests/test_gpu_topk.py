"""GPU parity of the router's per-row top-k (SLA2 page, section 2.B: the top-k block scores of
each query block, ties to the lowest index) in every regime of the library's kernels: keys
held in registers at 8, 12, 16, 20, 24 and 32 per lane (switching above 512, 768, 1024,
1280 and 1536 key blocks) and the radix kernel beyond 2048 key blocks.

Two cases per key-block count: a ragged last block with ordinary scores (selections equal to
the oracle's, near ties only valid), and every block duplicated so that each score occurs
twice. With an odd k the k-th score is then tied with its twin, the search cannot stop early,
and the lower index must win: selections bit-identical to the oracle's, every row.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from oracle import sla_oracle as so             # noqa: E402
from workloads import make_custom               # noqa: E402
from tests.gpu_helpers import to_device, check_masks  # noqa: E402

NBKS = [512, 513, 768, 769, 1024, 1025, 1280, 1281, 1536, 1537, 2048, 2049]


@pytest.fixture(scope="module")
def sla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_linear_hybrid_amd as s
    return s


def oracle_routes(x, top_k):
    p = x.problem
    pq, pk = x.proj_q.astype(np.float64), x.proj_k.astype(np.float64)
    return [[so.route_head(x.as_f64("q")[b, h], x.as_f64("k")[b, h], pq, pk, p.block, top_k)
             for h in range(p.heads)] for b in range(p.batch)]


@pytest.mark.parametrize("nbk", NBKS)
def test_topk_ragged(sla, nbk):
    x = make_custom(1, 2, 64 * 3 - 5, 64 * nbk - 7, 64, 1, dtype="bf16", kind="normal",
                    seed=nbk)
    q, k, v, pq, pk, al = to_device(x)
    for top_k in (1, nbk // 3, nbk - 1):
        print(f"top-k ragged: nbk={nbk} k={top_k}", flush=True)
        idx = sla.sla_route(q, k, pq, pk, top_k).cpu().numpy()
        check_masks(idx, oracle_routes(x, top_k), top_k)


@pytest.mark.parametrize("nbk", NBKS)
def test_topk_paired_ties(sla, nbk):
    x = make_custom(1, 1, 64 * 4, 64 * nbk, 64, 1, dtype="bf16", kind="normal", seed=nbk + 1)
    kk = x.k[0, 0]
    half = nbk // 2
    kk[64 * half:64 * 2 * half] = kk[:64 * half]      # block half + j repeats block j
    q, k, v, pq, pk, al = to_device(x)
    for top_k in (37, 38):
        print(f"top-k paired ties: nbk={nbk} k={top_k}", flush=True)
        idx = sla.sla_route(q, k, pq, pk, top_k).cpu().numpy()
        ref = oracle_routes(x, top_k)[0][0]
        assert np.array_equal(idx[0, 0], ref.idx)
        if top_k % 2 == 1 and nbk % 2 == 0:   # every score paired: the k-th is tied
            assert ref.near_tie.all()
