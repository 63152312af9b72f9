"""Stream behaviour of the forwards, which enqueue all their work on the caller's stream.

Checked: graph capture of each forward, and of the backward, replays bit-identically to the
eager call (several replays, with eager library work and synchronisations between them; the
library records no memset nodes); forwards on two caller streams at once give the results each gives
alone; the profiled entry point writes exactly what the plain one writes, for every variant;
junk in one head does not reach another head's output (ragged last blocks).
"""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from workloads import make_custom                       # noqa: E402
from tests.gpu_helpers import to_device                  # noqa: E402


@pytest.fixture(scope="module")
def sla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_linear_hybrid_amd as s
    return s


VARIANTS = ["sla", "fp8", "taylor", "pisa"]


def inputs(seed, nq=512, nkv=1100, d=128, top_k=4):
    x = make_custom(1, 2, nq, nkv, d, top_k, dtype="bf16", kind="smooth", seed=seed)
    return x, to_device(x)


def runner(sla, variant, dev, top_k):
    """make(tensors) -> (call, out): a forward of one variant into a preallocated workspace
    and output ``out``."""
    def make(tensors):
        q, k, v, pq, pk, al = tensors
        p = sla.make_problem(q, k, top_k)
        kind = {"fp8": sla.VARIANT_FP8, "pisa": sla.VARIANT_PISA}.get(variant,
                                                                      sla.VARIANT_FORWARD)
        ws = torch.empty(sla.workspace_size(p, kind), dtype=torch.uint8, device=dev)
        out = torch.empty(q.shape, dtype=torch.float32, device=dev)

        def call():
            if variant == "sla":
                sla.sla_forward(q, k, v, pq, pk, al, top_k, return_idx=False, workspace=ws,
                                out=out)
            elif variant == "fp8":
                sla.sla_forward_fp8(q, k, v, pq, pk, al, top_k, return_idx=False,
                                    workspace=ws, out=out)
            elif variant == "taylor":
                sla.sla_forward_taylor(q, k, v, al, top_k, return_idx=False, workspace=ws,
                                       out=out)
            else:
                sla.sla_forward_pisa(q, k, v, pq, pk, top_k, return_idx=False, workspace=ws,
                                     out=out)
        return call, out
    return make


@pytest.mark.parametrize("variant", VARIANTS)
def test_graph_replay_matches_eager(sla, variant):
    dev = torch.device("cuda")
    x, t = inputs(101)
    call, out = runner(sla, variant, dev, x.problem.top_k)(t)
    print(f"graph capture: {variant}", flush=True)
    call()
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    # other library work between replays, on the default stream
    _, t2 = inputs(202)
    other, _ = runner(sla, variant, dev, x.problem.top_k)(t2)
    for rep in range(3):
        call()                          # eager call on the captured buffers
        other()
        torch.cuda.synchronize()
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"


@pytest.mark.parametrize("variant", ["sla", "fp8"])
def test_two_caller_streams(sla, variant):
    dev = torch.device("cuda")
    (x1, t1), (x2, t2) = inputs(303), inputs(404, nq=700, nkv=900)
    c1, o1 = runner(sla, variant, dev, x1.problem.top_k)(t1)
    c2, o2 = runner(sla, variant, dev, x2.problem.top_k)(t2)
    c1()
    c2()
    torch.cuda.synchronize()
    alone1, alone2 = o1.clone(), o2.clone()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    print(f"two streams: {variant}", flush=True)
    for _ in range(3):
        with torch.cuda.stream(s1):
            c1()
        with torch.cuda.stream(s2):
            c2()
        torch.cuda.synchronize()
        assert torch.equal(o1, alone1)
        assert torch.equal(o2, alone2)


@pytest.mark.parametrize("variant", VARIANTS)
def test_profiled_matches_plain(sla, variant):
    dev = torch.device("cuda")
    x, t = inputs(505)
    q, k, v, pq, pk, al = t
    top_k = x.problem.top_k
    call, out = runner(sla, variant, dev, top_k)(t)
    call()
    torch.cuda.synchronize()
    plain = out.clone()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(sla.STAGES))]
    for e in evs:
        e.record()                      # torch creates the HIP event on its first record
    torch.cuda.synchronize()
    handles = (ctypes.c_void_p * len(evs))(*[e.cuda_event for e in evs])
    prof = sla.sla_forward_profiled(q, k, v, pq, pk, al, top_k, handles,
                                    fp8=variant == "fp8", taylor=variant == "taylor",
                                    pisa=variant == "pisa")
    torch.cuda.synchronize()
    assert torch.equal(prof, plain)
    times = [evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(len(sla.STAGES))]
    assert all(np.isfinite(times)) and min(times) >= 0.0


@pytest.mark.parametrize("variant", VARIANTS)
def test_heads_are_isolated_with_ragged_blocks(sla, variant):
    """Ragged last blocks (n_q = 200, n_kv = 130): in memory, the rows after a head's last
    token are the next head's. Replacing one head's Q, K and V by large finite junk must leave
    the other head's output unchanged bit for bit (each head in turn)."""
    dev = torch.device("cuda")
    x = make_custom(1, 2, 200, 130, 128, 2, dtype="bf16", kind="normal", seed=61)
    t = to_device(x)
    call, out = runner(sla, variant, dev, 2)(t)
    call()
    torch.cuda.synchronize()
    base = out.clone()
    gen = torch.Generator().manual_seed(7)
    for h_junk, h_keep in ((1, 0), (0, 1)):
        q, k, v = (a.clone() for a in t[:3])
        for a in (q, k, v):
            junk = torch.randn(a[0, h_junk].shape, generator=gen) * 300.0
            a[0, h_junk] = junk.to(dtype=a.dtype, device=dev)
        call2, out2 = runner(sla, variant, dev, 2)((q, k, v) + tuple(t[3:]))
        call2()
        torch.cuda.synchronize()
        assert torch.equal(out2[0, h_keep], base[0, h_keep]), (variant, h_keep)


def test_binding_refuses_mismatched_tensors(sla):
    """Checks that the C ABI cannot make: dtypes, shapes and devices of every tensor."""
    x = make_custom(1, 2, 128, 256, 64, 2, dtype="bf16", kind="normal", seed=3)
    q, k, v, pq, pk, al = to_device(x)
    bad = [
        ({"v": v.float()}, "v must match k"),
        ({"v": v[:, :, :128].contiguous()}, "v must match k"),
        ({"pq": pq.double()}, "proj"),
        ({"pk": pk[:32].contiguous()}, "proj"),
        ({"al": al[:1].contiguous()}, "alpha"),
        ({"al": al.cpu()}, "alpha is on"),
        ({"out": torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)}, "out must be"),
    ]
    for change, msg in bad:
        a = {"v": v, "pq": pq, "pk": pk, "al": al, "out": None}
        a.update(change)
        with pytest.raises(ValueError, match=msg):
            sla.sla_forward(q, k, a["v"], a["pq"], a["pk"], a["al"], 2, out=a["out"])
    with pytest.raises(TypeError, match="k has dtype"):
        sla.sla_forward(q, k.float(), v.float(), pq, pk, al, 2)


def test_backward_graph_replay_matches_eager(sla):
    """sla_backward captured in a graph replays bit-identically to the eager call (outputs and
    workspace preallocated, called through the C ABI), with other library work between the
    replays."""
    dev = torch.device("cuda")
    x, (q, k, v, pq, pk, al) = inputs(505, nq=450, nkv=900)
    top_k = x.problem.top_k
    _, idx = sla.sla_forward(q, k, v, pq, pk, al, top_k)
    dout = torch.randn(q.shape, device=dev, generator=torch.Generator(device=dev).manual_seed(2))
    p = sla.make_problem(q, k, top_k)
    ws = torch.empty(sla.sla_backward_workspace_size(p), dtype=torch.uint8, device=dev)
    grads = [torch.empty(q.shape, dtype=torch.float32, device=dev),
             torch.empty(k.shape, dtype=torch.float32, device=dev),
             torch.empty(v.shape, dtype=torch.float32, device=dev),
             torch.empty(al.shape, dtype=torch.float32, device=dev)]
    lib = sla.library()
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())   # noqa: E731

    def call():
        st = lib.sla_backward(ctypes.byref(p), ptr(q), ptr(k), ptr(v), ptr(al), ptr(dout),
                              ptr(idx), *(ptr(g_) for g_ in grads), ptr(ws),
                              ctypes.c_size_t(ws.numel()),
                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == 0
    call()
    torch.cuda.synchronize()
    eager = [g_.clone() for g_ in grads]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    _, t2 = inputs(606)
    other, _ = runner(sla, "sla", dev, top_k)(t2)
    for rep in range(3):
        call()
        other()
        torch.cuda.synchronize()
        for g_ in grads:
            g_.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("dq", "dk", "dv", "dalpha"), grads, eager):
            assert torch.equal(got, want), f"replay {rep}: {name}"
