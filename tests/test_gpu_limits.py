"""GPU parity at the size limits: the smallest shapes (one partial query block of 5 rows
against one partial key block of 10 keys), and the largest key-block count the library
accepts (8064 blocks of 64 keys, the row of 64-bit keys that top-k holds in 64 KB of LDS),
with a ragged last block.

At the largest size the complement walks its bitmap in several windows with more than 64 KB of
LDS, the piecewise tail's bitmap is full, and the router scores 8064 blocks per row. Masks
must equal the oracle's; outputs are compared on sampled rows (first and ragged last query
block) within the bf16 / fp8 bars.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle                                     # noqa: E402
from oracle import pisa as op                     # noqa: E402
from workloads import make_custom                 # noqa: E402
from tests.gpu_helpers import to_device, check_masks, max_err_over_rms  # noqa: E402

TOL, TOL_FP8 = 2e-2, 6e-2
MAX_BLOCKS = 8064


@pytest.fixture(scope="module")
def sla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_linear_hybrid_amd as s
    return s


@pytest.fixture(scope="module")
def big():
    """One head, 20 query blocks (the last one 57 rows), 8064 key blocks (the last one 44
    keys), top-k 40, smooth-field queries and keys."""
    return make_custom(1, 1, 64 * 20 - 7, MAX_BLOCKS * 64 - 20, 128, 40, dtype="bf16",
                       kind="smooth", seed=99)


def rows_of(p):
    return np.concatenate([np.arange(0, 64), np.arange((p.nbq - 1) * 64, p.n_q)])


def gpu(sla, x, fn):
    q, k, v, pq, pk, al = to_device(x)
    top_k = x.problem.top_k
    if fn == "pisa":
        out, idx = sla.sla_forward_pisa(q, k, v, pq, pk, top_k)
    elif fn == "fp8":
        out, idx = sla.sla_forward_fp8(q, k, v, pq, pk, al, top_k)
    else:
        out, idx = sla.sla_forward(q, k, v, pq, pk, al, top_k)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), idx.cpu().numpy()


@pytest.mark.slow
@pytest.mark.parametrize("fn", ["sla", "fp8", "pisa"])
def test_maximum_key_blocks(sla, big, fn):
    p = big.problem
    assert p.nbk == MAX_BLOCKS
    print(f"maximum key blocks: {fn} nq={p.n_q} nkv={p.n_kv}", flush=True)
    out, idx = gpu(sla, big, fn)
    rows, near = check_masks(idx, oracle.sla_oracle.route_full(big), p.top_k)
    rws = rows_of(p)
    if fn == "pisa":
        ref, _ = op.forward(big, heads=[(0, 0)], rows=rws)
    elif fn == "fp8":
        ref, _ = oracle.forward_fp8(big, heads=[(0, 0)], rows=rws)
    else:
        ref, _ = oracle.forward(big, heads=[(0, 0)], rows=rws)
    err, _ = max_err_over_rms(out[0, 0, rws], ref[0, 0, rws])
    print(f"  rows={rows} near_tie={near} max-abs/rms {err:.3e}")
    assert err <= (TOL_FP8 if fn == "fp8" else TOL)


@pytest.mark.slow
def test_maximum_key_blocks_d64(sla):
    """d = 64, two heads, normal inputs, fewer query blocks than the score tile (few-rows
    scoring)."""
    x = make_custom(1, 2, 64 * 6 - 30, MAX_BLOCKS * 64 - 1, 64, 64, dtype="bf16",
                    kind="normal", seed=101)
    p = x.problem
    out, idx = gpu(sla, x, "sla")
    check_masks(idx, oracle.sla_oracle.route_full(x), p.top_k)
    rws = rows_of(p)
    refs, gots = [], []
    for h in range(2):
        ref, _ = oracle.forward(x, heads=[(0, h)], rows=rws)
        refs.append(ref[0, h, rws])
        gots.append(out[0, h, rws])
    err, _ = max_err_over_rms(np.concatenate(gots), np.concatenate(refs))
    print(f"maximum key blocks d=64: max-abs/rms {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("fn", ["sla", "fp8", "pisa"])
@pytest.mark.parametrize("top_k", [0, 1])
def test_single_partial_blocks(sla, fn, top_k):
    """5 queries, 10 keys: one partial block each. top_k = 0 leaves everything to the linear
    branch (or the tail); top_k = 1 routes the only block (empty complement / tail)."""
    x = make_custom(1, 2, 5, 10, 64, top_k, dtype="bf16", kind="normal", seed=7 + top_k)
    out, idx = gpu(sla, x, fn)
    assert idx.shape == (1, 2, 1, top_k) and (top_k == 0 or np.all(idx == 0))
    if fn == "pisa":
        ref, _ = op.forward(x)
    elif fn == "fp8":
        ref, _ = oracle.forward_fp8(x)
    else:
        ref, _ = oracle.forward(x)
    err, _ = max_err_over_rms(out, ref)
    print(f"single partial blocks {fn} top_k={top_k}: max-abs/rms {err:.3e}")
    assert err <= (TOL_FP8 if fn == "fp8" else TOL)
