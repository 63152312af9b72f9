"""GPU parity of the allocation-free decode entry point (sla_forward_cached_noalloc).

It must give what sla_forward_cached gives on the same inputs (it runs the same kernels on
the same workspace layout, so bit for bit), and both must meet the oracle's bar (masks
exact, output within 2e-2 x RMS). Two calls in a row on one GPU, the second on a smaller
problem, so the second runs on the array the first one left behind.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle                                   # noqa: E402
from workloads import make_custom               # noqa: E402
from tests.gpu_helpers import to_device, check_masks, max_err_over_rms  # noqa: E402

TOL = 2e-2


@pytest.fixture(scope="module")
def sla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_linear_hybrid_amd as s
    return s


def test_noalloc_matches_cached_forward_on_two_calls(sla):
    cases = [(2, 4, 130, 5000, 128, 9, "smooth", 71),   # larger first
             (1, 2, 64, 700, 64, 3, "normal", 72)]      # then smaller, ragged
    for B, H, nq, nkv, d, top_k, kind, seed in cases:
        print(f"noalloc case B={B} H={H} nq={nq} nkv={nkv} d={d} k={top_k} {kind}", flush=True)
        x = make_custom(B, H, nq, nkv, d, top_k, dtype="bf16", kind=kind, seed=seed)
        q, k, v, pq, pk, al = to_device(x)
        cache = torch.empty(sla.kv_cache_size(sla.make_problem(k, k, 0)), dtype=torch.uint8,
                            device="cuda")
        sla.sla_kv_cache_update(k, v, pk, cache)
        ref_out, ref_idx = sla.sla_forward_cached(q, k, v, pq, al, top_k, cache)
        out = torch.full_like(ref_out, float("nan"))
        idx = torch.full_like(ref_idx, -1)
        sla.sla_forward_cached_noalloc(q, k, v, pq, al, top_k, cache, out, idx)
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_idx)
        assert torch.equal(out, ref_out)
        got = out.cpu().numpy().astype(np.float64)
        check_masks(idx.cpu().numpy(), oracle.sla_oracle.route_full(x), top_k)
        ref, _ = oracle.forward(x)
        err, _ = max_err_over_rms(got, ref)
        print(f"  max-abs/rms {err:.3e}", flush=True)
        assert err <= TOL


def test_noalloc_without_index_output(sla):
    """block_idx = NULL keeps the selection in the scratch array; the output is unchanged."""
    x = make_custom(1, 3, 100, 2000, 128, 5, dtype="bf16", kind="smooth", seed=73)
    q, k, v, pq, pk, al = to_device(x)
    cache = torch.empty(sla.kv_cache_size(sla.make_problem(k, k, 0)), dtype=torch.uint8,
                        device="cuda")
    sla.sla_kv_cache_update(k, v, pk, cache)
    ref_out, _ = sla.sla_forward_cached(q, k, v, pq, al, 5, cache)
    out = torch.empty_like(ref_out)
    sla.sla_forward_cached_noalloc(q, k, v, pq, al, 5, cache, out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out)


def test_noalloc_rejects_a_problem_beyond_the_scratch_array(sla):
    """A problem whose workspace would exceed the fixed array is refused before anything is
    enqueued (SLA_ERR_SCRATCH), and the binding raises SlaError; out is left untouched."""
    B, H, nq, nkv, d, top_k = 1, 16, 16384, 1024, 128, 4
    q = torch.zeros((B, H, nq, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, H, nkv, d), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(k)
    p = sla.make_problem(q, k, top_k)
    assert sla.cached_workspace_size(p) > sla.NOALLOC_SCRATCH_BYTES
    pq = torch.eye(d, dtype=torch.float32, device="cuda")
    al = torch.full((H, d), 0.5, dtype=torch.float32, device="cuda")
    cache = torch.zeros(sla.kv_cache_size(sla.make_problem(k, k, 0)), dtype=torch.uint8,
                        device="cuda")
    out = torch.full((B, H, nq, d), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(sla.SlaError) as exc:
        sla.sla_forward_cached_noalloc(q, k, v, pq, al, top_k, cache, out)
    assert exc.value.status == 9
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
