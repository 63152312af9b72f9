"""Out-of-bounds canaries: every forward entry point, the router, the cached forward and the
backward are called through the C ABI with their outputs, block indices and workspace placed
inside larger buffers whose other bytes hold a sentinel pattern. After the call the sentinel
bytes before and after each region must be untouched (no write past a buffer), at ragged
shapes (partial last query and key blocks) and both head dims."""
import ctypes

import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from workloads import make_custom              # noqa: E402
from tests.gpu_helpers import to_device        # noqa: E402

GUARD = 4096          # sentinel bytes on each side of a region (a multiple of 256)
SENTINEL = 0xA5


@pytest.fixture(scope="module")
def sla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_linear_hybrid_amd as s
    return s


class Guarded:
    """`nbytes` usable bytes at a 256-aligned offset inside a sentinel-filled uint8 buffer."""

    def __init__(self, nbytes):
        self.nbytes = int(nbytes)
        self.buf = torch.full((self.nbytes + 2 * GUARD,), SENTINEL, dtype=torch.uint8,
                              device="cuda")

    @property
    def ptr(self):
        return ctypes.c_void_p(self.buf.data_ptr() + GUARD)

    def intact(self):
        head = self.buf[:GUARD]
        tail = self.buf[GUARD + self.nbytes:]
        return bool((head == SENTINEL).all()) and bool((tail == SENTINEL).all())


def vp(t):
    return ctypes.c_void_p(t.data_ptr())


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


SHAPES = [
    # B, H, nq, nkv, d, top_k
    (1, 2, 200, 333, 128, 3),
    (2, 1, 130, 470, 64, 2),
    (1, 2, 100, 16400, 128, 5),     # few query blocks over many key blocks: the cache path
]


def inputs(sla, B, H, nq, nkv, d, top_k, out_dtype=torch.float32):
    x = make_custom(B, H, nq, nkv, d, top_k, dtype="bf16", kind="smooth", seed=nq + nkv + d)
    q, k, v, pq, pk, al = to_device(x)
    p = sla.make_problem(q, k, top_k, out_dtype=out_dtype)
    nbq = -(-nq // 64)
    return x, (q, k, v, pq, pk, al), p, nbq


@pytest.mark.parametrize("B,H,nq,nkv,d,top_k", SHAPES)
@pytest.mark.parametrize("entry", ["sla_forward", "sla_forward_bf16out", "sla_forward_fp8",
                                   "sla_forward_taylor", "sla_forward_pisa", "sla_route"])
def test_forward_entry_points_write_only_their_buffers(sla, entry, B, H, nq, nkv, d, top_k):
    print(f"canaries {entry} B={B} H={H} nq={nq} nkv={nkv} d={d} k={top_k}", flush=True)
    out_dtype = torch.bfloat16 if entry == "sla_forward_bf16out" else torch.float32
    _, (q, k, v, pq, pk, al), p, nbq = inputs(sla, B, H, nq, nkv, d, top_k, out_dtype)
    variant = {"sla_forward_fp8": sla.VARIANT_FP8, "sla_forward_pisa": sla.VARIANT_PISA,
               "sla_forward_taylor": sla.VARIANT_TAYLOR}.get(entry, sla.VARIANT_FORWARD)
    ws = Guarded(sla.workspace_size(p, variant))
    out = Guarded(B * H * nq * d * (2 if out_dtype == torch.bfloat16 else 4))
    idx = Guarded(B * H * nbq * top_k * 4)
    lib = sla.library()
    P = ctypes.byref(p)
    W = (ws.ptr, ctypes.c_size_t(ws.nbytes), stream())
    if entry in ("sla_forward", "sla_forward_bf16out", "sla_forward_fp8"):
        name = "sla_forward_fp8" if entry == "sla_forward_fp8" else "sla_forward"
        st = getattr(lib, name)(P, vp(q), vp(k), vp(v), vp(pq), vp(pk), vp(al), out.ptr, idx.ptr,
                                *W)
    elif entry == "sla_forward_taylor":
        st = lib.sla_forward_taylor(P, vp(q), vp(k), vp(v), vp(al), out.ptr, idx.ptr, *W)
    elif entry == "sla_forward_pisa":
        st = lib.sla_forward_pisa(P, vp(q), vp(k), vp(v), vp(pq), vp(pk), out.ptr, idx.ptr, *W)
    else:
        st = lib.sla_route(P, vp(q), vp(k), vp(pq), vp(pk), idx.ptr, *W)
    assert st == 0, sla.STATUS.get(st, st)
    torch.cuda.synchronize()
    assert ws.intact(), "workspace guard overwritten"
    assert idx.intact(), "block_idx guard overwritten"
    assert out.intact(), "output guard overwritten"
    # the regions themselves were written (indices in range, output finite)
    got = idx.buf[GUARD:GUARD + idx.nbytes].view(torch.int32)
    if top_k:
        assert int(got.min()) >= 0 and int(got.max()) < -(-nkv // 64)
    if entry != "sla_route":
        o = out.buf[GUARD:GUARD + out.nbytes].view(out_dtype)
        assert bool(torch.isfinite(o.float()).all())


@pytest.mark.parametrize("B,H,nq,nkv,d,top_k", SHAPES[:2])
def test_cached_forward_and_cache_update_write_only_their_buffers(sla, B, H, nq, nkv, d, top_k):
    _, (q, k, v, pq, pk, al), p, nbq = inputs(sla, B, H, nq, nkv, d, top_k)
    lib = sla.library()
    pk0 = sla.make_problem(k, k, 0)
    cache = Guarded(sla.kv_cache_size(pk0))
    cws = Guarded(int(lib.sla_kv_cache_workspace_size(ctypes.byref(pk0), 0)))
    st = lib.sla_kv_cache_update(ctypes.byref(pk0), vp(k), vp(v), vp(pk), 0, cache.ptr, cws.ptr,
                                 ctypes.c_size_t(cws.nbytes), stream())
    assert st == 0, sla.STATUS.get(st, st)
    ws = Guarded(sla.cached_workspace_size(p))
    out = Guarded(B * H * nq * d * 4)
    idx = Guarded(B * H * nbq * top_k * 4)
    st = lib.sla_forward_cached(ctypes.byref(p), vp(q), vp(k), vp(v), vp(pq), vp(al), cache.ptr,
                                out.ptr, idx.ptr, ws.ptr, ctypes.c_size_t(ws.nbytes), stream())
    assert st == 0, sla.STATUS.get(st, st)
    torch.cuda.synchronize()
    for name, g in (("cache", cache), ("cache workspace", cws), ("workspace", ws),
                    ("block_idx", idx), ("output", out)):
        assert g.intact(), f"{name} guard overwritten"


@pytest.mark.parametrize("B,H,nq,nkv,d,top_k", SHAPES[:2])
def test_backward_writes_only_its_buffers(sla, B, H, nq, nkv, d, top_k):
    _, (q, k, v, pq, pk, al), p, nbq = inputs(sla, B, H, nq, nkv, d, top_k)
    _, sel = sla.sla_forward(q, k, v, pq, pk, al, top_k)
    dout = torch.randn(q.shape, device="cuda", generator=torch.Generator("cuda").manual_seed(1))
    lib = sla.library()
    ws = Guarded(sla.sla_backward_workspace_size(p))
    dq = Guarded(q.numel() * 4)
    dk = Guarded(k.numel() * 4)
    dv = Guarded(v.numel() * 4)
    dal = Guarded(H * d * 4)
    st = lib.sla_backward(ctypes.byref(p), vp(q), vp(k), vp(v), vp(al), vp(dout), vp(sel),
                          dq.ptr, dk.ptr, dv.ptr, dal.ptr, ws.ptr, ctypes.c_size_t(ws.nbytes),
                          stream())
    assert st == 0, sla.STATUS.get(st, st)
    torch.cuda.synchronize()
    for name, g in (("workspace", ws), ("dq", dq), ("dk", dk), ("dv", dv), ("dalpha", dal)):
        assert g.intact(), f"{name} guard overwritten"
