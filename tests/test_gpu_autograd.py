"""The torch.autograd wrapper (sla_attention): its forward is sla_forward's output bit for
bit, its backward hands back sla_backward's gradients at the forward's selection (cast to
the inputs' dtypes), and the router's projections get no gradient."""
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


@pytest.mark.parametrize("fp8", [False, True])
def test_autograd_wrapper_matches_the_entry_points(sla, fp8):
    x = make_custom(1, 2, 300, 700, 128, 3, dtype="bf16", kind="smooth", seed=41)
    q, k, v, pq, pk, al = to_device(x)
    leaves = [t.detach().clone().requires_grad_(True) for t in (q, k, v, al)]
    out, idx = sla.sla_attention(leaves[0], leaves[1], leaves[2], pq, pk, leaves[3], 3, fp8=fp8,
                                 return_idx=True)
    fwd = sla.sla_forward_fp8 if fp8 else sla.sla_forward
    want_out, want_idx = fwd(q, k, v, pq, pk, al, 3)
    assert torch.equal(idx, want_idx) and torch.equal(out, want_out)
    g = torch.from_numpy(np.random.default_rng(3).standard_normal(q.shape).astype(np.float32)).cuda()
    (out * g).sum().backward()
    dq, dk, dv, dal = sla.sla_backward(q, k, v, al, g, want_idx)
    torch.cuda.synchronize()
    for got, want in zip(leaves, (dq, dk, dv, dal)):
        assert got.grad is not None and got.grad.dtype == got.dtype
        assert torch.equal(got.grad, want.to(got.dtype))
    assert pq.grad is None and pk.grad is None
