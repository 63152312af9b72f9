"""Repeated calls give identical bits (the library promises bit-reproducible results: no
floating-point atomics, fixed reduction orders), checked on shapes large enough that many
workgroups run concurrently and each streams many blocks: the router's pooled, projected
queries and keys (through the block scores they produce) and the key/value summary cache."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from workloads import make_custom               # noqa: E402
from tests.gpu_helpers import to_device         # noqa: E402


@pytest.fixture(scope="module")
def sla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_linear_hybrid_amd as s
    return s


def test_router_scores_are_bit_reproducible(sla):
    x = make_custom(1, 8, 64 * 300 - 7, 64 * 300, 128, 10, dtype="bf16", kind="smooth", seed=91)
    q, k, v, pq, pk, al = to_device(x)
    prob = sla.make_problem(q, k, 10)
    ws = torch.zeros(sla.workspace_size(prob, sla.VARIANT_FORWARD), dtype=torch.uint8,
                     device="cuda")
    off, size = sla.workspace_region(prob, "scores")
    runs = []
    for _ in range(4):
        out, idx = sla.sla_forward(q, k, v, pq, pk, al, 10, workspace=ws)
        torch.cuda.synchronize()
        runs.append((ws[off:off + size].clone(), out.clone(), idx.clone()))
    for s_, o_, i_ in runs[1:]:
        assert torch.equal(s_, runs[0][0])
        assert torch.equal(o_, runs[0][1]) and torch.equal(i_, runs[0][2])


def test_summary_cache_is_bit_reproducible(sla):
    x = make_custom(2, 4, 64, 64 * 600 + 17, 128, 8, dtype="bf16", kind="normal", seed=92)
    q, k, v, pq, pk, al = to_device(x)
    p = sla.make_problem(k, k, 0)
    caches = []
    for _ in range(4):
        c = torch.zeros(sla.kv_cache_size(p), dtype=torch.uint8, device="cuda")
        sla.sla_kv_cache_update(k, v, pk, c)
        torch.cuda.synchronize()
        caches.append(c)
    for c in caches[1:]:
        assert torch.equal(c, caches[0])
