"""Host-side tests of the C ABI: symbols, validation and workspace sizing.

No compute is launched here: every call below is rejected by argument validation, which
runs before anything is enqueued, so the fake device addresses are never dereferenced.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sla.h")

sla = pytest.importorskip("sparse_linear_hybrid_amd")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sla.LIB_PATH):
        pytest.fail("libsla.so is not built (run __graft_entry__.build())")
    return sla.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sla_\w+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    names = declared_functions()
    for n in ("sla_route", "sla_forward", "sla_forward_fp8", "sla_workspace_size",
              "sla_status_string", "sla_forward_profiled"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(sla.EXPORTS) == set(declared_functions())


def prob(**kw):
    base = dict(batch=1, heads=2, n_q=300, n_kv=700, head_dim=128, block=64, top_k=3,
                in_dtype=1, out_dtype=0)
    base.update(kw)
    return sla.Problem(**base)


FAKE = 0x100000          # aligned, never dereferenced (every call fails validation first)
MISALIGNED = 0x100004


def call_forward(lib, p, q=FAKE, k=FAKE, v=FAKE, pq=FAKE, pk=FAKE, al=FAKE, o=FAKE, idx=None,
                 ws=FAKE, ws_bytes=0, fn="sla_forward"):
    vp = ctypes.c_void_p
    pp = ctypes.byref(p) if p is not None else None
    return getattr(lib, fn)(pp, vp(q), vp(k), vp(v), vp(pq), vp(pk), vp(al), vp(o), vp(idx),
                            vp(ws), ctypes.c_size_t(ws_bytes), vp(0))


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), "SLA_ERR_SHAPE"), (dict(n_q=0), "SLA_ERR_SHAPE"),
    (dict(n_kv=-5), "SLA_ERR_SHAPE"), (dict(in_dtype=7), "SLA_ERR_DTYPE"),
    (dict(out_dtype=3), "SLA_ERR_DTYPE"), (dict(head_dim=96), "SLA_ERR_UNSUPPORTED"),
    (dict(block=32), "SLA_ERR_UNSUPPORTED"), (dict(top_k=-1), "SLA_ERR_TOPK"),
    (dict(top_k=12), "SLA_ERR_TOPK"), (dict(n_kv=64 * 8065), "SLA_ERR_UNSUPPORTED"),
])
def test_problem_validation(lib, kw, status):
    code = {v: k for k, v in sla.sla.STATUS.items()}[status]
    assert call_forward(lib, prob(**kw)) == code
    assert lib.sla_workspace_size(ctypes.byref(prob(**kw)), 0) == 0


def test_pointer_validation(lib):
    p = prob()
    assert call_forward(lib, None) == 1
    assert call_forward(lib, p, q=0) == 1
    assert call_forward(lib, p, al=0) == 1
    assert call_forward(lib, p, o=MISALIGNED) == 5
    assert call_forward(lib, p, idx=MISALIGNED) == 5
    # valid problem and pointers but no / too small workspace
    assert call_forward(lib, p, ws=0, ws_bytes=1 << 40) == 6
    need = lib.sla_workspace_size(ctypes.byref(p), 0)
    assert call_forward(lib, p, ws_bytes=need - 1) == 6
    # the fp8 entry point accepts only bf16 inputs
    assert call_forward(lib, prob(in_dtype=0), fn="sla_forward_fp8") == 3
    assert call_forward(lib, p, fn="sla_forward_fp8", ws_bytes=need) == 6   # fp8 needs more


def test_route_validation(lib):
    vp = ctypes.c_void_p
    p = prob()
    r = lib.sla_route(ctypes.byref(p), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(0), vp(FAKE),
                      ctypes.c_size_t(1 << 30), vp(0))
    assert r == 1    # block_idx is required
    r = lib.sla_route(ctypes.byref(p), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE),
                      ctypes.c_size_t(0), vp(0))
    assert r == 6


def test_workspace_size_monotone(lib):
    def ws(**kw):
        return lib.sla_workspace_size(ctypes.byref(prob(**kw)), 0)
    base = ws()
    assert base > 0
    assert ws(n_q=3000) > base and ws(n_kv=7000) > base and ws(heads=4) > base
    assert lib.sla_workspace_size(ctypes.byref(prob()), 1) > base


def test_status_strings(lib):
    for code in range(10):
        assert lib.sla_status_string(code).decode()
    assert lib.sla_status_string(99) == b"unknown status"


def test_stage_names_follow_header_enum():
    text = open(HEADER).read()
    vals = {m.group(1).lower(): int(m.group(2))
            for m in re.finditer(r"SLA_STAGE_(\w+)\s*=\s*(\d+)", text)}
    n = int(re.search(r"SLA_NUM_STAGES\s*=\s*(\d+)", text).group(1))
    assert sorted(vals.values()) == list(range(n))
    assert tuple(sorted(vals, key=vals.get)) == sla.STAGES


def test_workspace_regions_follow_header_enum(lib):
    text = open(HEADER).read()
    vals = {m.group(1).lower(): int(m.group(2))
            for m in re.finditer(r"SLA_WS_(\w+)\s*=\s*(\d+)", text)}
    assert vals == dict(sla.WS_REGIONS)


def test_kv_cache_layout_and_growth(lib):
    """The cache is S_tot^T, z_tot, then k~ block-major: its size grows only with the number
    of key blocks, by B*H*d*8 bytes per block."""
    def size(**kw):
        return lib.sla_kv_cache_size(ctypes.byref(prob(**kw)))
    BH, d = 2, 128
    base = size(n_kv=640)
    stot = BH * d * d * 4
    ztot_end = -(-stot // 256) * 256 + BH * d * 4
    assert base == -(-ztot_end // 256) * 256 + 10 * BH * d * 8
    assert size(n_kv=641) - base == BH * d * 8
    assert size(n_kv=700) == size(n_kv=704)
    assert size(n_kv=0) == 0


def test_kv_cache_update_validation(lib):
    vp = ctypes.c_void_p
    p = prob(n_kv=700)

    def upd(prob_=p, n_done=0, k=FAKE, cache=FAKE, ws=FAKE, ws_bytes=1 << 30):
        return lib.sla_kv_cache_update(ctypes.byref(prob_), vp(k), vp(FAKE), vp(FAKE),
                                       ctypes.c_int32(n_done), vp(cache), vp(ws),
                                       ctypes.c_size_t(ws_bytes), vp(0))
    assert upd(prob_=prob(in_dtype=0)) == 3            # bf16 only
    assert upd(n_done=-1) == 2 and upd(n_done=701) == 2
    assert upd(k=0) == 1 and upd(cache=0) == 1
    assert upd(cache=MISALIGNED) == 5
    need = lib.sla_kv_cache_workspace_size(ctypes.byref(p), 0)
    assert need >= 256
    assert upd(ws_bytes=need - 1) == 6
    assert lib.sla_kv_cache_workspace_size(ctypes.byref(p), 701) == 0
    # an update near the end touches only the last key blocks: smaller partial totals
    big = prob(n_kv=64 * 200)
    assert (lib.sla_kv_cache_workspace_size(ctypes.byref(big), 64 * 199) <
            lib.sla_kv_cache_workspace_size(ctypes.byref(big), 0))


def test_forward_cached_validation(lib):
    vp = ctypes.c_void_p
    p = prob()

    def fwd(prob_=p, q=FAKE, cache=FAKE, ws_bytes=1 << 40, idx=None):
        return lib.sla_forward_cached(ctypes.byref(prob_), vp(q), vp(FAKE), vp(FAKE), vp(FAKE),
                                      vp(FAKE), vp(cache), vp(FAKE), vp(idx), vp(FAKE),
                                      ctypes.c_size_t(ws_bytes), vp(0))
    assert fwd(prob_=prob(in_dtype=0)) == 3
    assert fwd(prob_=prob(top_k=12)) == 4
    assert fwd(q=0) == 1 and fwd(cache=0) == 1
    assert fwd(idx=MISALIGNED) == 5
    need = lib.sla_cached_workspace_size(ctypes.byref(p))
    assert need > 0 and fwd(ws_bytes=need - 1) == 6


def test_forward_cached_noalloc_validation(lib):
    """The allocation-free entry point validates like sla_forward_cached and refuses, before
    any device call, a problem whose decode workspace exceeds its fixed scratch array."""
    vp = ctypes.c_void_p

    def fwd(prob_, q=FAKE):
        pp = ctypes.byref(prob_) if prob_ is not None else None
        return lib.sla_forward_cached_noalloc(pp, vp(q), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE),
                                              vp(FAKE), vp(FAKE), vp(None), vp(0))
    assert fwd(None) == 1
    assert fwd(prob(top_k=12)) == 4
    assert fwd(prob(head_dim=96)) == 7
    big = prob(batch=4, heads=32, n_q=64 * 16, n_kv=131072, top_k=64)
    assert lib.sla_cached_workspace_size(ctypes.byref(big)) > sla.NOALLOC_SCRATCH_BYTES
    assert fwd(big) == 9
    decode = prob(batch=4, heads=32, n_q=64, n_kv=131072, top_k=64)
    assert 0 < lib.sla_cached_workspace_size(ctypes.byref(decode)) <= sla.NOALLOC_SCRATCH_BYTES
    hdr = open(HEADER).read()
    assert "#define SLA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)" in hdr
    assert sla.NOALLOC_SCRATCH_BYTES == 128 << 20


def test_backward_validation(lib):
    vp = ctypes.c_void_p

    def bwd(prob_, q=FAKE, idx=FAKE, ws=FAKE, ws_bytes=1 << 40):
        pp = ctypes.byref(prob_) if prob_ is not None else None
        return lib.sla_backward(pp, vp(q), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(idx),
                                vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(ws),
                                ctypes.c_size_t(ws_bytes), vp(0))
    p = prob()
    assert bwd(None) == 1
    assert bwd(prob(in_dtype=0)) == 3
    assert bwd(prob(top_k=12)) == 4
    assert bwd(p, q=0) == 1 and bwd(p, idx=0) == 1
    assert bwd(p, idx=MISALIGNED) == 5
    need = lib.sla_backward_workspace_size(ctypes.byref(p))
    assert need > lib.sla_workspace_size(ctypes.byref(p), 0)
    assert bwd(p, ws_bytes=need - 1) == 6 and bwd(p, ws=0) == 6
    assert lib.sla_backward_workspace_size(ctypes.byref(prob(head_dim=96))) == 0


def test_taylor_entry_points_validation(lib):
    vp = ctypes.c_void_p
    p = prob()
    need = lib.sla_workspace_size(ctypes.byref(p), 0)
    r = lib.sla_route_taylor(ctypes.byref(p), vp(FAKE), vp(FAKE), vp(0), vp(FAKE),
                             ctypes.c_size_t(need), vp(0))
    assert r == 1    # block_idx is required
    r = lib.sla_route_taylor(ctypes.byref(prob(top_k=12)), vp(FAKE), vp(FAKE), vp(FAKE),
                             vp(FAKE), ctypes.c_size_t(need), vp(0))
    assert r == 4

    def fwd(prob_=p, q=FAKE, al=FAKE, ws_bytes=need):
        return lib.sla_forward_taylor(ctypes.byref(prob_), vp(q), vp(FAKE), vp(FAKE), vp(al),
                                      vp(FAKE), vp(None), vp(FAKE), ctypes.c_size_t(ws_bytes),
                                      vp(0))
    assert fwd(q=0) == 1 and fwd(al=0) == 1
    assert fwd(ws_bytes=need - 1) == 6
    assert fwd(prob_=prob(head_dim=96)) == 7


@pytest.mark.parametrize("flags", [3, 5, 6, 8, -1])
def test_profiled_rejects_unknown_flags(lib, flags):
    vp = ctypes.c_void_p
    p = prob()
    need = lib.sla_workspace_size(ctypes.byref(p), 1)
    r = lib.sla_forward_profiled(ctypes.byref(p), *[vp(FAKE)] * 7, vp(None), vp(FAKE),
                                 ctypes.c_size_t(need), vp(0), flags, vp(None))
    assert r == 7


def test_workspace_variants(lib):
    """Variants 0 .. 3 have their own sizes; anything else is invalid (size 0)."""
    p = prob()
    sizes = [lib.sla_workspace_size(ctypes.byref(p), v) for v in (0, 1, 2, 3)]
    assert all(s > 0 for s in sizes)
    assert sizes[0] == sizes[3]           # no cache path here: Taylor shares the layout
    assert lib.sla_workspace_size(ctypes.byref(p), 4) == 0
    assert lib.sla_workspace_size(ctypes.byref(p), -1) == 0
    text = open(HEADER).read()
    vals = {m.group(1): int(m.group(2))
            for m in re.finditer(r"SLA_VARIANT_(\w+)\s*=\s*(\d+)", text)}
    assert vals == {"FORWARD": sla.VARIANT_FORWARD, "FP8": sla.VARIANT_FP8,
                    "PISA": sla.VARIANT_PISA, "TAYLOR": sla.VARIANT_TAYLOR}


def test_workspace_regions_by_variant(lib):
    """fp8 regions exist only in the fp8 layout, piecewise regions only in the piecewise one,
    and the complement regions not in the piecewise one."""
    p = prob()
    off, size = ctypes.c_size_t(), ctypes.c_size_t()

    def region(variant, name):
        return lib.sla_workspace_region(ctypes.byref(p), variant, sla.WS_REGIONS[name],
                                        ctypes.byref(off), ctypes.byref(size))
    assert region(1, "q8") == 0 and region(0, "q8") == 2 and region(2, "q8") == 2
    assert region(2, "hbar") == 0 and region(0, "hbar") == 2 and region(1, "hbar") == 2
    assert region(0, "sc") == 0 and region(2, "sc") == 2
    assert region(2, "scores") == 0 and region(5, "scores") == 2
    total = lib.sla_workspace_size(ctypes.byref(p), 2)
    for name in ("hbar", "cent_hi", "cent_lo", "vsum"):
        assert region(2, name) == 0
        assert off.value % 256 == 0 and off.value + size.value <= total
    d, BH = p.head_dim, p.batch * p.heads
    npad = -(-(-(-p.n_kv // 64)) // 64) * 64
    region(2, "vsum")
    assert size.value == BH * d * npad * 2
    region(2, "hbar")
    assert size.value == BH * d * d * 2


def test_cache_path_workspace(lib):
    """A chunk of at most 8 query blocks per head against at least 256 key blocks (bf16) takes
    the cache path: its forward workspace is the summary cache, the update's partial totals
    and the cached forward's workspace, far below the per-key-block layout that the Taylor
    forward keeps; the scores and complement regions do not exist there."""
    few = prob(batch=4, heads=32, n_q=64, n_kv=131072, top_k=64)
    fwd = lib.sla_workspace_size(ctypes.byref(few), 0)
    taylor = lib.sla_workspace_size(ctypes.byref(few), 3)
    cache = lib.sla_kv_cache_size(ctypes.byref(few))
    dec = lib.sla_cached_workspace_size(ctypes.byref(few))
    upd = lib.sla_kv_cache_workspace_size(ctypes.byref(few), 0)
    assert cache + dec + upd <= fwd <= cache + dec + upd + 3 * 256
    # the routers share the forward variant: their buffers (pooled, projected Q and K,
    # scores, indices, key variances) fit as well
    small = prob(batch=1, heads=2, n_q=64 * 3, n_kv=64 * 512, top_k=1, head_dim=64)
    BH, d, nbq, nbk = 2, 64, 3, 512
    al = lambda x: -(-x // 256) * 256                     # noqa: E731
    route = al(BH * nbq * d * 8) + al(BH * nbk * d * 8) + al(BH * nbq * nbk * 8) \
        + al(BH * nbq * 1 * 4) + al(BH * nbk * d * 8)
    assert lib.sla_workspace_size(ctypes.byref(small), 0) >= route
    assert taylor > 10 * fwd
    off, size = ctypes.c_size_t(), ctypes.c_size_t()
    for name, want in (("sc", 7), ("zc", 7), ("scores", 7)):
        assert lib.sla_workspace_region(ctypes.byref(few), 0, sla.WS_REGIONS[name],
                                        ctypes.byref(off), ctypes.byref(size)) == want
        assert lib.sla_workspace_region(ctypes.byref(few), 3, sla.WS_REGIONS[name],
                                        ctypes.byref(off), ctypes.byref(size)) == 0
    # fp32 inputs, more query blocks or fewer key blocks keep the per-block layout
    for kw in (dict(in_dtype=0), dict(n_q=64 * 9), dict(n_kv=64 * 255)):
        p = prob(batch=4, heads=32, n_q=kw.get("n_q", 64), n_kv=kw.get("n_kv", 131072),
                 top_k=64, in_dtype=kw.get("in_dtype", 1))
        assert lib.sla_workspace_size(ctypes.byref(p), 0) == lib.sla_workspace_size(
            ctypes.byref(p), 3)


def test_pisa_validation(lib):
    vp = ctypes.c_void_p
    p = prob()
    need = lib.sla_workspace_size(ctypes.byref(p), 2)

    def fwd(prob_=p, q=FAKE, pq=FAKE, o=FAKE, ws=FAKE, ws_bytes=need, idx=None):
        return lib.sla_forward_pisa(ctypes.byref(prob_), vp(q), vp(FAKE), vp(FAKE), vp(pq),
                                    vp(FAKE), vp(o), vp(idx), vp(ws), ctypes.c_size_t(ws_bytes),
                                    vp(0))
    assert fwd(q=0) == 1 and fwd(pq=0) == 1 and fwd(o=0) == 1
    assert fwd(ws_bytes=need - 1) == 6
    assert fwd(ws=MISALIGNED) == 5 and fwd(idx=MISALIGNED) == 5
    assert fwd(prob_=prob(head_dim=96)) == 7
    assert fwd(prob_=prob(top_k=12)) == 4


def test_mfma_rate_validation(lib):
    """The throughput diagnostic rejects a NULL sink and empty launches before enqueuing."""
    fn = lib.sla_diag_mfma_rate
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    assert fn(None, 512, 16, None) == 1                      # SLA_ERR_NULL
    assert fn(ctypes.c_void_p(FAKE), 0, 16, None) == 2       # SLA_ERR_SHAPE
    assert fn(ctypes.c_void_p(FAKE), 512, 0, None) == 2
