"""GPU parity: the HIP path (through the C ABI) against the CPU float64 oracle.

Masks must match bit for bit (ties to the lowest index); outputs within max-abs error
<= 2e-2 x RMS of the oracle output (fp32 output). Small cases span several tiles and ragged
tails; the named workloads are checked at full size (masks in full, outputs on sampled
query blocks that the oracle evaluates one by one).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle                                   # noqa: E402
from oracle import sla_oracle as so             # noqa: E402
from workloads import make_custom, make_inputs, bf16_bits_to_f32  # noqa: E402
from tests.gpu_helpers import to_device, check_masks, max_err_over_rms  # noqa: E402

TOL = 2e-2


@pytest.fixture(scope="module")
def sla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_linear_hybrid_amd as s
    return s


def run_forward(sla, x, out_dtype=torch.float32):
    q, k, v, pq, pk, al = to_device(x)
    out, idx = sla.sla_forward(q, k, v, pq, pk, al, x.problem.top_k, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), idx.cpu().numpy()


CASES = [
    # B, H, nq, nkv, d, top_k, dtype, kind
    (1, 2, 256, 256, 64, 2, "bf16", "normal"),
    (1, 2, 300, 300, 128, 3, "bf16", "smooth"),        # ragged tail (300 = 4*64 + 44)
    (2, 1, 200, 520, 128, 4, "bf16", "smooth"),        # n_q != n_kv, both ragged
    (1, 3, 192, 192, 64, 3, "f32", "normal"),
    (1, 1, 64, 1000, 128, 5, "bf16", "normal"),        # one query block, many key blocks
    (1, 2, 130, 130, 128, 1, "bf16", "normal"),        # last blocks hold 2 tokens
]


@pytest.mark.parametrize("B,H,nq,nkv,d,top_k,dtype,kind", CASES)
def test_forward_small(sla, B, H, nq, nkv, d, top_k, dtype, kind):
    x = make_custom(B, H, nq, nkv, d, top_k, dtype=dtype, kind=kind, seed=nq + d)
    print(f"case B={B} H={H} nq={nq} nkv={nkv} d={d} k={top_k} {dtype} {kind}", flush=True)
    out, idx = run_forward(sla, x)
    ref, ref_idx = oracle.forward(x)
    check_masks(idx, oracle.sla_oracle.route_full(x), top_k)
    err, rms = max_err_over_rms(out, ref)
    assert err <= TOL, f"max-abs/rms {err:.3e}"


@pytest.mark.parametrize("top_k", [0, 1])
def test_degenerate_selection_counts(sla, top_k):
    """top_k = 0 (pure linear branch) and a single block."""
    x = make_custom(1, 2, 256, 320, 128, top_k, dtype="bf16", kind="normal", seed=5)
    out, idx = run_forward(sla, x)
    ref, _ = oracle.forward(x)
    assert idx.shape[-1] == top_k
    err, _ = max_err_over_rms(out, ref)
    assert err <= TOL


def test_all_blocks_alpha_one_is_dense(sla):
    """top_k = all key blocks, alpha = 1: dense softmax attention; the empty complement
    must contribute exactly nothing."""
    x = make_custom(1, 2, 320, 448, 128, 7, dtype="bf16", kind="normal", seed=9)
    x.alpha[:] = 1.0
    out, idx = run_forward(sla, x)
    q, k, v = (torch.from_numpy(x.as_f64(n)) for n in ("q", "k", "v"))
    dense = torch.nn.functional.scaled_dot_product_attention(q, k, v).numpy()
    assert np.all(idx == np.arange(7))
    err, _ = max_err_over_rms(out, dense)
    assert err <= TOL


def test_topk0_alpha0_is_linear(sla):
    x = make_custom(1, 2, 192, 256, 64, 0, dtype="f32", kind="normal", seed=11)
    x.alpha[:] = 0.0
    out, _ = run_forward(sla, x)
    ref, _ = oracle.forward(x)
    err, _ = max_err_over_rms(out, ref)
    assert err <= TOL


@pytest.mark.parametrize("alpha_value", [0.0, None])
def test_one_block_left_out(sla, alpha_value):
    """top_k = Nbk - 1: each query block's complement is a single key block, so z_c and S_c
    are the smallest they can be without being empty (z_c = z_tot minus nearly all of it);
    alpha = 0 leaves the linear branch alone in the output."""
    x = make_custom(1, 2, 300, 640, 128, 9, dtype="bf16", kind="smooth", seed=17)
    if alpha_value is not None:
        x.alpha[:] = alpha_value
    out, idx = run_forward(sla, x)
    ref, _ = oracle.forward(x)
    check_masks(idx, oracle.sla_oracle.route_full(x), 9)
    err, _ = max_err_over_rms(out, ref)
    print(f"top_k = Nbk - 1, alpha {alpha_value}: max-abs/rms {err:.3e}", flush=True)
    assert err <= TOL


def test_bf16_output_matches_fp32_output(sla):
    x = make_custom(1, 2, 256, 256, 128, 2, dtype="bf16", kind="smooth", seed=3)
    o32, i32 = run_forward(sla, x, torch.float32)
    o16, i16 = run_forward(sla, x, torch.bfloat16)
    assert np.array_equal(i32, i16)
    want = torch.from_numpy(o32).to(torch.bfloat16).float().numpy()
    assert np.array_equal(o16, want)


def test_route_entry_point(sla):
    x = make_custom(2, 2, 200, 700, 128, 4, dtype="bf16", kind="smooth", seed=21)
    q, k, v, pq, pk, al = to_device(x)
    idx = sla.sla_route(q, k, pq, pk, 4).cpu().numpy()
    check_masks(idx, oracle.sla_oracle.route_full(x), 4)


def test_planted_ties_lowest_index(sla):
    """Duplicated key blocks tie exactly; the lower block index must win."""
    x = make_custom(1, 1, 128, 512, 64, 2, dtype="bf16", kind="normal", seed=4)
    k = x.k[0, 0]
    for src, dst in [(1, 5), (2, 6), (3, 7)]:
        k[dst * 64:(dst + 1) * 64] = k[src * 64:(src + 1) * 64]
    q, kk, v, pq, pk, al = to_device(x)
    idx = sla.sla_route(q, kk, pq, pk, 2).cpu().numpy()
    ref = oracle.sla_oracle.route_full(x)
    # exact ties are resolved identically on both sides: require bit equality everywhere
    assert np.array_equal(idx[0, 0], ref[0][0].idx)
    assert ref[0][0].near_tie.any(), "the planted duplicates should create boundary ties"


@pytest.mark.parametrize("boost", [0.0, 6.0, 40.0])
def test_max_rises_inside_a_tile(sla, boost):
    """Keys 32..63 of every key block lean towards the queries, so the running maximum jumps
    between the two halves of a tile (by more than the rescale slack for the larger boosts)
    as well as between tiles; the online softmax must stay exact in every case."""
    from workloads import Inputs, bf16_round_bits
    x = make_custom(1, 2, 256, 384, 128, 3, dtype="bf16", kind="normal", seed=17)
    q = x.as_f64("q")
    k = x.as_f64("k")
    for h in range(2):
        u = q[0, h].mean(axis=0)
        u /= np.linalg.norm(u)
        second = (np.arange(k.shape[2]) % 64) >= 32
        k[0, h, second] += boost * u
    k_bits = bf16_round_bits(k.astype(np.float32))
    y = Inputs(x.problem, x.q, k_bits, x.v, x.proj_q, x.proj_k, x.alpha, dict(x.meta))
    out, idx = run_forward(sla, y)
    ref, _ = oracle.forward(y)
    check_masks(idx, oracle.sla_oracle.route_full(y), 3)
    err, _ = max_err_over_rms(out, ref)
    print(f"  boost {boost}: max-abs/rms {err:.3e}")
    assert err <= TOL, f"max-abs/rms {err:.3e}"


def test_deterministic(sla):
    x = make_custom(1, 2, 256, 256, 128, 3, dtype="bf16", kind="smooth", seed=8)
    a, ia = run_forward(sla, x)
    b, ib = run_forward(sla, x)
    assert np.array_equal(a, b) and np.array_equal(ia, ib)


# ----------------------------------------------------------------------------- workloads
def _sampled_check(sla, x, blocks_per_head=3, heads=None, seed=0, no_ties=False):
    out, idx = run_forward(sla, x)
    routes = oracle.sla_oracle.route_full(x)
    rows, near = check_masks(idx, routes, x.problem.top_k)
    if no_ties:      # the workloads hold no boundary ties: every row must match exactly
        assert near == 0, f"{near} rows needed the near-tie allowance"
    p = x.problem
    rng = np.random.default_rng(seed)
    pairs = heads or [(b, h) for b in range(p.batch) for h in range(p.heads)]
    errs = []
    refs = []
    gots = []
    for b, h in pairs:
        blocks = rng.choice(p.nbq, size=min(blocks_per_head, p.nbq), replace=False)
        if p.nbq > 1 and (p.nbq - 1) not in blocks:
            blocks[-1] = p.nbq - 1          # always include the ragged last block
        rws = np.concatenate([np.arange(i * 64, min(i * 64 + 64, p.n_q)) for i in blocks])
        ref, _ = oracle.forward(x, heads=[(b, h)], rows=rws)
        refs.append(ref[b, h, rws])
        gots.append(out[b, h, rws])
    ref = np.concatenate(refs)
    got = np.concatenate(gots)
    err, rms = max_err_over_rms(got, ref)
    print(f"{p.name}: rows={rows} near_tie={near} max-abs/rms={err:.3e} rms={rms:.4f}")
    assert err <= TOL


@pytest.mark.parametrize("d", [64, 128])
def test_grouped_launch_ragged_group(sla, d):
    """Enough query blocks that neighbouring blocks share a workgroup (133 blocks per head:
    the last group holds one active block), checked on sampled blocks incl. the last."""
    x = make_custom(1, 12, 64 * 132 + 30, 1500, d, 5, dtype="bf16", kind="smooth", seed=40 + d)
    _sampled_check(sla, x, blocks_per_head=3, heads=[(0, 0), (0, 11)])


def test_single_block_groups_many_workgroups(sla):
    """640 query blocks in all (below the grouping threshold, so one query block per
    workgroup): more workgroups than the GPU holds at once, bf16 and fp32 inputs."""
    for dtype in ("bf16", "f32"):
        x = make_custom(1, 8, 64 * 80 - 20, 512, 128, 3, dtype=dtype, kind="smooth", seed=47)
        _sampled_check(sla, x, blocks_per_head=3, heads=[(0, 1), (0, 7)])


def test_tiny_workload(sla):
    x = make_inputs("tiny")
    out, idx = run_forward(sla, x)
    ref, ref_idx = oracle.forward(x)
    assert np.array_equal(idx, ref_idx)
    err, _ = max_err_over_rms(out, ref)
    print(f"tiny: max-abs/rms {err:.3e}", flush=True)
    assert err <= TOL


@pytest.mark.slow
def test_video95_full(sla):
    x = make_inputs("video95")
    _sampled_check(sla, x, blocks_per_head=2, heads=[(0, 0), (0, 5), (0, 11)], no_ties=True)


@pytest.mark.slow
def test_video90_full(sla):
    x = make_inputs("video90")
    _sampled_check(sla, x, blocks_per_head=2, heads=[(0, 0), (0, 39)], no_ties=True)


@pytest.mark.slow
def test_longctx_full(sla):
    x = make_inputs("longctx")
    _sampled_check(sla, x, blocks_per_head=1, heads=[(0, 0), (3, 31)], no_ties=True)


# ----------------------------------------------------------------------------- fp8 branch
TOL_FP8 = 6e-2


def run_forward_fp8(sla, x, out_dtype=torch.float32):
    q, k, v, pq, pk, al = to_device(x)
    out, idx = sla.sla_forward_fp8(q, k, v, pq, pk, al, x.problem.top_k, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), idx.cpu().numpy()


FP8_CASES = [
    (1, 2, 256, 256, 128, 2, "smooth"),
    (1, 2, 300, 300, 128, 3, "smooth"),     # ragged tail
    (2, 1, 200, 520, 64, 4, "normal"),      # d = 64, n_q != n_kv
    (1, 1, 64, 1000, 128, 5, "normal"),
]


@pytest.mark.parametrize("B,H,nq,nkv,d,top_k,kind", FP8_CASES)
def test_fp8_small(sla, B, H, nq, nkv, d, top_k, kind):
    x = make_custom(B, H, nq, nkv, d, top_k, dtype="bf16", kind=kind, seed=nq + 3 * d)
    print(f"fp8 case B={B} H={H} nq={nq} nkv={nkv} d={d} k={top_k} {kind}", flush=True)
    out, idx = run_forward_fp8(sla, x)
    ref, ref_idx = oracle.forward_fp8(x)
    check_masks(idx, oracle.sla_oracle.route_full(x), top_k)
    err, rms = max_err_over_rms(out, ref)
    # information only: distance from the unquantised forward and from the literal reading
    e_exact, _ = max_err_over_rms(out, oracle.forward(x)[0])
    e_lit, _ = max_err_over_rms(out, oracle.fp8.forward_fp8_literal(x)[0])
    print(f"  max-abs/rms {err:.3e} (vs unquantised {e_exact:.3e}, vs literal reading {e_lit:.3e})")
    assert err <= TOL_FP8, f"max-abs/rms {err:.3e}"


def test_fp8_masks_equal_bf16_masks(sla):
    x = make_custom(1, 2, 320, 448, 128, 3, dtype="bf16", kind="smooth", seed=12)
    _, i8 = run_forward_fp8(sla, x)
    _, i16 = run_forward(sla, x)
    assert np.array_equal(i8, i16)


@pytest.mark.slow
def test_video95_fp8_full(sla):
    x = make_inputs("video95_fp8")
    out, idx = run_forward_fp8(sla, x)
    routes = oracle.sla_oracle.route_full(x)
    rows, near = check_masks(idx, routes, x.problem.top_k)
    assert near == 0
    rng = np.random.default_rng(1)
    p = x.problem
    refs, gots, exact, lit = [], [], [], []
    for h in (0, 7, 11):
        blocks = rng.choice(p.nbq, size=2, replace=False)
        rws = np.concatenate([np.arange(i * 64, i * 64 + 64) for i in blocks])
        ref, _ = oracle.forward_fp8(x, heads=[(0, h)], rows=rws)
        refs.append(ref[0, h, rws])
        gots.append(out[0, h, rws])
        exact.append(oracle.forward(x, heads=[(0, h)], rows=rws)[0][0, h, rws])
        lit.append(oracle.fp8.forward_fp8_literal(x, heads=[(0, h)], rows=rws)[0][0, h, rws])
    got = np.concatenate(gots)
    err, rms = max_err_over_rms(got, np.concatenate(refs))
    e_exact, _ = max_err_over_rms(got, np.concatenate(exact))
    e_lit, _ = max_err_over_rms(got, np.concatenate(lit))
    print(f"video95_fp8: rows={rows} near_tie={near} max-abs/rms={err:.3e} rms={rms:.4f} "
          f"(vs unquantised {e_exact:.3e}, vs literal reading {e_lit:.3e})")
    assert err <= TOL_FP8


def _v8_key_order():
    """Key stored at each byte position of a V8 tile row (the P8 operand order)."""
    order = np.empty(64, np.int64)
    for hh in range(2):
        for slot in range(32):
            order[32 * hh + slot] = 32 * (slot // 16) + 8 * ((slot % 16) // 4) + 4 * hh + slot % 4
    return order


@pytest.mark.parametrize("nq,nkv,d", [(256, 320, 128), (200, 130, 64)])
def test_fp8_quantiser_bit_exact(sla, nq, nkv, d):
    """E4M3 values and block exponents of Q, K, V equal the oracle's quantisation exactly
    (Q and K are held as bf16, V as E4M3 bytes)."""
    from oracle import fp8 as ofp8
    x = make_custom(1, 2, nq, nkv, d, 2, dtype="bf16", kind="smooth", seed=31)
    q, k, v, pq, pk, al = to_device(x)
    prob = sla.make_problem(q, k, 2)
    ws = torch.zeros(sla.workspace_size(prob, True), dtype=torch.uint8, device="cuda")
    sla.sla_forward_fp8(q, k, v, pq, pk, al, 2, workspace=ws)
    torch.cuda.synchronize()
    wsh = ws.cpu().numpy()

    def region(name, dtype):
        off, size = sla.workspace_region(prob, name, sla.VARIANT_FP8)
        return wsh[off:off + size].view(dtype)

    nbq, nbk = prob.n_q // 64 + (prob.n_q % 64 > 0), -(-nkv // 64)
    q8 = region("q8", np.uint16).reshape(2, nbq * 64, d)
    k8 = region("k8", np.uint16).reshape(2, nbk * 64, d)
    v8 = region("v8", np.uint8).reshape(2, nbk, d, 64)
    eq = region("eq", np.int32).reshape(2, nbq)
    ek = region("ek", np.int32).reshape(2, nbk)
    ev = region("ev", np.int32).reshape(2, nbk)
    order = _v8_key_order()
    for h in range(2):
        for name, g8, ge, n in (("q", q8, eq, nq), ("k", k8, ek, nkv)):
            want, s = ofp8.quantise_blocks(x.as_f64(name)[0, h], 64)
            assert np.array_equal(ge[h], np.log2(s).astype(np.int32)), name
            assert np.array_equal(bf16_bits_to_f32(g8[h, :n]).astype(np.float64), want), name
            assert not g8[h, n:].any()
        want, s = ofp8.quantise_blocks(x.as_f64("v")[0, h], 64)
        assert np.array_equal(ev[h], np.log2(s).astype(np.int32))
        got = np.zeros((nbk * 64, d))
        for j in range(nbk):
            got[j * 64 + order] = ofp8.e4m3_decode(v8[h, j]).T
        assert np.array_equal(got[:nkv], want)
