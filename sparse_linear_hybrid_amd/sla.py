"""ctypes binding of libsla.so (include/sla.h).

Argument marshalling only: tensors are passed as device pointers, the current torch stream
as the HIP stream, and every step of the computation runs in the library's HIP kernels.
Device memory for outputs and the workspace is allocated with torch (the library itself
never allocates). There is no fallback: the library is loaded on first use and a missing
library raises ImportError there.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsla.so")

SLA_F32, SLA_BF16 = 0, 1
STATUS = {0: "SLA_OK", 1: "SLA_ERR_NULL", 2: "SLA_ERR_SHAPE", 3: "SLA_ERR_DTYPE",
          4: "SLA_ERR_TOPK", 5: "SLA_ERR_ALIGN", 6: "SLA_ERR_WORKSPACE",
          7: "SLA_ERR_UNSUPPORTED", 8: "SLA_ERR_HIP", 9: "SLA_ERR_SCRATCH"}
EXPORTS = ("sla_workspace_size", "sla_route", "sla_forward", "sla_forward_fp8",
           "sla_forward_profiled", "sla_workspace_region", "sla_status_string",
           "sla_kv_cache_size", "sla_kv_cache_workspace_size", "sla_kv_cache_update",
           "sla_cached_workspace_size", "sla_forward_cached", "sla_route_taylor",
           "sla_forward_taylor", "sla_forward_pisa", "sla_forward_cached_noalloc",
           "sla_backward_workspace_size", "sla_backward", "sla_diag_fp8_mfma",
           "sla_diag_mfma_rate")
WS_REGIONS = {"q8": 0, "k8": 1, "v8": 2, "eq": 3, "ek": 4, "ev": 5, "scores": 6, "sc": 7, "zc": 8,
              "hbar": 9, "cent_hi": 10, "cent_lo": 11, "vsum": 12}
# workspace layouts (sla_workspace_size / sla_workspace_region)
VARIANT_FORWARD, VARIANT_FP8, VARIANT_PISA, VARIANT_TAYLOR = 0, 1, 2, 3
STAGES = ("kv_summary", "route", "complement", "quant", "sparse")
# flags of sla_forward_profiled
PROFILE_FP8 = 1
PROFILE_TAYLOR = 2
PROFILE_PISA = 4


class SlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} "
                         f"({library().sla_status_string(status).decode()})")


class Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("n_q", ctypes.c_int32),
                ("n_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("block", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m sparse_linear_hybrid_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32p = ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(ctypes.c_int32)
    pp = ctypes.POINTER(Problem)
    lib.sla_workspace_size.argtypes = [pp, ctypes.c_int]
    lib.sla_workspace_size.restype = sz
    lib.sla_route.argtypes = [pp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.sla_route.restype = ctypes.c_int
    lib.sla_forward_pisa.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.sla_forward_pisa.restype = ctypes.c_int
    for name in ("sla_forward", "sla_forward_fp8"):
        f = getattr(lib, name)
        f.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        f.restype = ctypes.c_int
    lib.sla_forward_profiled.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                         ctypes.c_int, vp]
    lib.sla_forward_profiled.restype = ctypes.c_int
    lib.sla_workspace_region.argtypes = [pp, ctypes.c_int, ctypes.c_int,
                                         ctypes.POINTER(ctypes.c_size_t),
                                         ctypes.POINTER(ctypes.c_size_t)]
    lib.sla_workspace_region.restype = ctypes.c_int
    lib.sla_status_string.argtypes = [ctypes.c_int]
    lib.sla_status_string.restype = ctypes.c_char_p
    lib.sla_kv_cache_size.argtypes = [pp]
    lib.sla_kv_cache_size.restype = sz
    lib.sla_kv_cache_workspace_size.argtypes = [pp, ctypes.c_int32]
    lib.sla_kv_cache_workspace_size.restype = sz
    lib.sla_kv_cache_update.argtypes = [pp, vp, vp, vp, ctypes.c_int32, vp, vp, sz, vp]
    lib.sla_kv_cache_update.restype = ctypes.c_int
    lib.sla_cached_workspace_size.argtypes = [pp]
    lib.sla_cached_workspace_size.restype = sz
    lib.sla_forward_cached.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.sla_diag_fp8_mfma.argtypes = [vp, vp, vp, vp, vp]
    lib.sla_diag_fp8_mfma.restype = ctypes.c_int
    lib.sla_diag_mfma_rate.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp]
    lib.sla_diag_mfma_rate.restype = ctypes.c_int
    lib.sla_backward_workspace_size.argtypes = [pp]
    lib.sla_backward_workspace_size.restype = sz
    lib.sla_backward.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.sla_backward.restype = ctypes.c_int
    lib.sla_forward_cached_noalloc.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.sla_forward_cached_noalloc.restype = ctypes.c_int
    lib.sla_forward_cached.restype = ctypes.c_int
    lib.sla_route_taylor.argtypes = [pp, vp, vp, vp, vp, sz, vp]
    lib.sla_route_taylor.restype = ctypes.c_int
    lib.sla_forward_taylor.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.sla_forward_taylor.restype = ctypes.c_int
    return lib


_LIB: Optional[ctypes.CDLL] = None


def library() -> ctypes.CDLL:
    """The loaded libsla.so (loaded on first use; raises ImportError if it is not built)."""
    global _LIB
    if _LIB is None:
        _LIB = _load()
    return _LIB


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return SLA_BF16
    if t == torch.float32:
        return SLA_F32
    raise TypeError(f"unsupported dtype {t}")


def make_problem(q: torch.Tensor, k: torch.Tensor, top_k: int, block: int = 64,
                 out_dtype: torch.dtype = torch.float32) -> Problem:
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [batch, heads, tokens, head_dim]")
    B, H, nq, d = q.shape
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != d:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)}")
    return Problem(B, H, nq, k.shape[2], d, block, top_k, _dtype_code(q.dtype),
                   _dtype_code(out_dtype))


def _check(q: torch.Tensor, k: torch.Tensor, v: Optional[torch.Tensor] = None,
           proj: Tuple[Optional[torch.Tensor], ...] = (), alpha: Optional[torch.Tensor] = None,
           out: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
           buffers: Tuple[Optional[torch.Tensor], ...] = ()) -> None:
    """Checks what the C ABI cannot see before anything is enqueued: every tensor is on the
    GPU that holds q, K and V share q's dtype (V has K's shape), projections are fp32
    [d, d], alpha is fp32 [heads, d], a caller's output has q's shape and out_dtype, and
    workspace or cache buffers are device tensors. Raises ValueError / TypeError."""
    if not q.is_cuda:
        raise ValueError("q must be a GPU tensor")
    dev = q.device
    B, H, _, d = q.shape
    named = [("k", k), ("v", v), ("alpha", alpha), ("out", out)]
    named += [(f"proj[{i}]", t) for i, t in enumerate(proj)]
    named += [(f"buffer[{i}]", t) for i, t in enumerate(buffers)]
    for name, t in named:
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, q on {dev}")
    if k.dtype != q.dtype:
        raise TypeError(f"k has dtype {k.dtype}, q {q.dtype}")
    if v is not None and (v.dtype != k.dtype or v.shape != k.shape):
        raise ValueError(f"v must match k: v {v.dtype}{tuple(v.shape)}, "
                         f"k {k.dtype}{tuple(k.shape)}")
    for i, t in enumerate(proj):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != (d, d)):
            raise ValueError(f"proj[{i}] must be float32 [{d}, {d}], got {t.dtype}{tuple(t.shape)}")
    if alpha is not None and (alpha.dtype != torch.float32 or tuple(alpha.shape) != (H, d)):
        raise ValueError(f"alpha must be float32 [{H}, {d}], got {alpha.dtype}"
                         f"{tuple(alpha.shape)}")
    if out is not None and (out.shape != q.shape or out.dtype != out_dtype):
        raise ValueError(f"out must be {out_dtype}{tuple(q.shape)}, got {out.dtype}"
                         f"{tuple(out.shape)}")


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def workspace_size(p: Problem, variant=VARIANT_FORWARD) -> int:
    """Workspace bytes for a layout: VARIANT_FORWARD (False), VARIANT_FP8 (True),
    VARIANT_PISA or VARIANT_TAYLOR."""
    return int(library().sla_workspace_size(ctypes.byref(p), int(variant)))


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _workspace(p: Problem, variant, device, workspace: Optional[torch.Tensor]) -> torch.Tensor:
    """The caller's workspace if it is large enough (any dtype; its bytes count), else a new
    uint8 tensor of the size the library asks for."""
    need = workspace_size(p, variant)
    if need == 0:
        raise SlaError(2, "sla_workspace_size")
    if workspace is None or _nbytes(workspace) < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    return workspace


def sla_route(q, k, proj_q, proj_k, top_k: int, block: int = 64,
              workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Router: int32 block indices [B, H, ceil(n_q/block), top_k], ascending per row."""
    p = make_problem(q, k, top_k, block)
    _check(q, k, proj=(proj_q, proj_k), buffers=(workspace,))
    ws = _workspace(p, VARIANT_FORWARD, q.device, workspace)
    idx = torch.empty((p.batch, p.heads, -(-p.n_q // block), top_k), dtype=torch.int32,
                      device=q.device)
    st = library().sla_route(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(proj_q), _ptr(proj_k),
                             _ptr(idx), _ptr(ws), ctypes.c_size_t(_nbytes(ws)), _stream(q.device))
    if st != 0:
        raise SlaError(st, "sla_route")
    return idx


def _forward(name: str, q, k, v, proj_q, proj_k, alpha, top_k: int, block: int,
             out_dtype: torch.dtype, return_idx: bool, workspace,
             out) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    p = make_problem(q, k, top_k, block, out_dtype)
    _check(q, k, v, (proj_q, proj_k), alpha, out, out_dtype, (workspace,))
    variant = VARIANT_FP8 if name == "sla_forward_fp8" else VARIANT_FORWARD
    ws = _workspace(p, variant, q.device, workspace)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    idx = None
    if return_idx:
        idx = torch.empty((p.batch, p.heads, -(-p.n_q // block), top_k), dtype=torch.int32,
                          device=q.device)
    st = getattr(library(), name)(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(proj_q),
                             _ptr(proj_k), _ptr(alpha), _ptr(out), _ptr(idx), _ptr(ws),
                             ctypes.c_size_t(_nbytes(ws)), _stream(q.device))
    if st != 0:
        raise SlaError(st, name)
    return out, idx


def sla_forward(q, k, v, proj_q, proj_k, alpha, top_k: int, block: int = 64,
                out_dtype: torch.dtype = torch.float32, return_idx: bool = True,
                workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None):
    """SLA2 forward (bf16 sparse branch). Returns (O, block_idx or None)."""
    return _forward("sla_forward", q, k, v, proj_q, proj_k, alpha, top_k, block, out_dtype,
                    return_idx, workspace, out)


def sla_forward_fp8(q, k, v, proj_q, proj_k, alpha, top_k: int, block: int = 64,
                    out_dtype: torch.dtype = torch.float32, return_idx: bool = True,
                    workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None):
    """SLA2 forward with the E4M3 sparse branch. Returns (O, block_idx or None)."""
    return _forward("sla_forward_fp8", q, k, v, proj_q, proj_k, alpha, top_k, block, out_dtype,
                    return_idx, workspace, out)


def sla_forward_profiled(q, k, v, proj_q, proj_k, alpha, top_k: int, events, fp8: bool = False,
                         block: int = 64, out_dtype: torch.dtype = torch.float32,
                         workspace: Optional[torch.Tensor] = None,
                         out: Optional[torch.Tensor] = None, taylor: bool = False,
                         pisa: bool = False):
    """sla_forward / sla_forward_fp8 / sla_forward_taylor (``taylor=True``: proj_q and proj_k
    are ignored) / sla_forward_pisa (``pisa=True``: alpha is ignored) that also records
    ``events`` (2 per stage, in the order of STAGES: before, after) on the current stream.
    ``events``: ctypes array of hipEvent_t handles created by the caller. Returns O."""
    if int(fp8) + int(taylor) + int(pisa) > 1:
        raise ValueError("fp8, taylor and pisa select different forward paths")
    p = make_problem(q, k, top_k, block, out_dtype)
    _check(q, k, v, () if taylor else (proj_q, proj_k), None if pisa else alpha, out,
           out_dtype, (workspace,))
    variant = (VARIANT_FP8 if fp8 else VARIANT_PISA if pisa else
               VARIANT_TAYLOR if taylor else VARIANT_FORWARD)
    ws = _workspace(p, variant, q.device, workspace)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    flags = PROFILE_FP8 if fp8 else (PROFILE_TAYLOR if taylor else (PROFILE_PISA if pisa else 0))
    pq = None if taylor else _ptr(proj_q)
    pk = None if taylor else _ptr(proj_k)
    al = None if pisa else _ptr(alpha)
    st = library().sla_forward_profiled(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), pq, pk, al,
                                        _ptr(out), None, _ptr(ws), ctypes.c_size_t(_nbytes(ws)),
                                        _stream(q.device), flags, events)
    if st != 0:
        raise SlaError(st, "sla_forward_profiled")
    return out


def workspace_region(p: Problem, name: str, variant=VARIANT_FORWARD) -> Tuple[int, int]:
    """(byte offset, byte size) of a named workspace region (see WS_REGIONS) in the layout
    of ``variant`` (False / True select the forward / fp8 layouts)."""
    off, size = ctypes.c_size_t(), ctypes.c_size_t()
    st = library().sla_workspace_region(ctypes.byref(p), int(variant), WS_REGIONS[name],
                                        ctypes.byref(off), ctypes.byref(size))
    if st != 0:
        raise SlaError(st, "sla_workspace_region")
    return off.value, size.value


# ----------------------------------------------------------------------------- summary cache
def kv_cache_size(p: Problem) -> int:
    """Bytes of the key/value summary cache for p.n_kv tokens (see include/sla.h)."""
    return int(library().sla_kv_cache_size(ctypes.byref(p)))


def sla_kv_cache_update(k, v, proj_k, cache: torch.Tensor, n_done: int = 0, block: int = 64,
                        workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Bring ``cache`` (uint8 device tensor of at least kv_cache_size bytes) from the first
    n_done tokens of k, v to all of them (n_done = 0 builds it). Returns ``cache``."""
    p = make_problem(k, k, 0, block)
    _check(k, k, v, (proj_k,), buffers=(cache, workspace))
    if _nbytes(cache) < kv_cache_size(p):
        raise ValueError("cache tensor too small")
    need = int(library().sla_kv_cache_workspace_size(ctypes.byref(p), int(n_done)))
    if need == 0:
        raise SlaError(2, "sla_kv_cache_workspace_size")
    if workspace is None or _nbytes(workspace) < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=k.device)
    st = library().sla_kv_cache_update(ctypes.byref(p), _ptr(k), _ptr(v), _ptr(proj_k),
                                       int(n_done), _ptr(cache), _ptr(workspace),
                                       ctypes.c_size_t(_nbytes(workspace)), _stream(k.device))
    if st != 0:
        raise SlaError(st, "sla_kv_cache_update")
    return cache


def cached_workspace_size(p: Problem) -> int:
    return int(library().sla_cached_workspace_size(ctypes.byref(p)))


def sla_forward_cached(q, k, v, proj_q, alpha, top_k: int, cache: torch.Tensor, block: int = 64,
                       out_dtype: torch.dtype = torch.float32, return_idx: bool = True,
                       workspace: Optional[torch.Tensor] = None,
                       out: Optional[torch.Tensor] = None):
    """SLA2 forward against a summary cache covering all of k, v. Returns (O, block_idx or
    None)."""
    p = make_problem(q, k, top_k, block, out_dtype)
    _check(q, k, v, (proj_q,), alpha, out, out_dtype, (cache, workspace))
    need = cached_workspace_size(p)
    if need == 0:
        raise SlaError(2, "sla_cached_workspace_size")
    if workspace is None or _nbytes(workspace) < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    idx = None
    if return_idx:
        idx = torch.empty((p.batch, p.heads, -(-p.n_q // block), top_k), dtype=torch.int32,
                          device=q.device)
    st = library().sla_forward_cached(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(proj_q),
                                      _ptr(alpha), _ptr(cache), _ptr(out), _ptr(idx),
                                      _ptr(workspace), ctypes.c_size_t(_nbytes(workspace)),
                                      _stream(q.device))
    if st != 0:
        raise SlaError(st, "sla_forward_cached")
    return out, idx


NOALLOC_SCRATCH_BYTES = 128 << 20


def sla_forward_cached_noalloc(q, k, v, proj_q, alpha, top_k: int, cache: torch.Tensor,
                               out: torch.Tensor, block_idx: Optional[torch.Tensor] = None,
                               block: int = 64):
    """sla_forward_cached with the library's fixed scratch array instead of a workspace: the
    caller passes preallocated `out` (and optionally `block_idx`); nothing is allocated on
    the device by this call. Returns (out, block_idx)."""
    p = make_problem(q, k, top_k, block, out.dtype)
    _check(q, k, v, (proj_q,), alpha, out, out.dtype, (cache,))
    if block_idx is not None:
        want = (p.batch, p.heads, -(-p.n_q // block), top_k)
        if tuple(block_idx.shape) != want or block_idx.dtype != torch.int32 \
                or block_idx.device != q.device or not block_idx.is_contiguous():
            raise ValueError(f"block_idx must be a contiguous int32 {want} tensor on {q.device}")
    st = library().sla_forward_cached_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v),
                                              _ptr(proj_q), _ptr(alpha), _ptr(cache), _ptr(out),
                                              _ptr(block_idx), _stream(q.device))
    if st != 0:
        raise SlaError(st, "sla_forward_cached_noalloc")
    return out, block_idx


# ----------------------------------------------------------------------------- backward
def sla_backward_workspace_size(p: Problem) -> int:
    """Bytes of device workspace sla_backward needs for problem p (p.top_k = the selection's
    width, p.out_dtype = dout's dtype code)."""
    need = int(library().sla_backward_workspace_size(ctypes.byref(p)))
    if need == 0:
        raise SlaError(2, "sla_backward_workspace_size")
    return need


def sla_backward(q, k, v, alpha, dout, block_idx, block: int = 64,
                 workspace: Optional[torch.Tensor] = None):
    """Gradients of sla_forward at the selection block_idx for the upstream gradient dout
    (O's shape, fp32 or bf16). Returns (dq, dk, dv, dalpha), fp32."""
    top_k = int(block_idx.shape[-1])
    p = make_problem(q, k, top_k, block, dout.dtype)
    _check(q, k, v, (), alpha, dout, dout.dtype, (workspace, block_idx))
    want = (p.batch, p.heads, -(-p.n_q // block), top_k)
    if tuple(block_idx.shape) != want or block_idx.dtype != torch.int32 \
            or not block_idx.is_contiguous():
        raise ValueError(f"block_idx must be a contiguous int32 {want} tensor")
    need = sla_backward_workspace_size(p)
    if workspace is None or _nbytes(workspace) < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    dk = torch.empty(k.shape, dtype=torch.float32, device=q.device)
    dv = torch.empty(v.shape, dtype=torch.float32, device=q.device)
    dal = torch.empty((p.heads, p.head_dim), dtype=torch.float32, device=q.device)
    st = library().sla_backward(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                _ptr(dout), _ptr(block_idx), _ptr(dq), _ptr(dk), _ptr(dv),
                                _ptr(dal), _ptr(workspace), ctypes.c_size_t(_nbytes(workspace)),
                                _stream(q.device))
    if st != 0:
        raise SlaError(st, "sla_backward")
    return dq, dk, dv, dal


def sla_diag_fp8_mfma(a: torch.Tensor, b: torch.Tensor):
    """Diagnostic: (C on the fp8 instruction, C on the bf16 instruction) for E4M3 code tensors
    a [32, 64] and b [64, 32] (uint8, on the GPU). Both fp32 [32, 32]."""
    if a.shape != (32, 64) or b.shape != (64, 32) or a.dtype != torch.uint8 \
            or b.dtype != torch.uint8 or not (a.is_cuda and b.is_cuda):
        raise ValueError("a: uint8 [32, 64], b: uint8 [64, 32], GPU tensors")
    a, b = a.contiguous(), b.contiguous()
    c8 = torch.empty((32, 32), dtype=torch.float32, device=a.device)
    c16 = torch.empty_like(c8)
    st = library().sla_diag_fp8_mfma(_ptr(a), _ptr(b), _ptr(c8), _ptr(c16), _stream(a.device))
    if st != 0:
        raise SlaError(st, "sla_diag_fp8_mfma")
    return c8, c16


def sla_diag_mfma_rate(device, blocks: int = 512, iters: int = 4096, repeats: int = 3) -> float:
    """Diagnostic: the bf16 matrix-instruction rate (TFLOP/s) this GPU reaches: the median of
    `repeats` timed launches of the throughput loop, after one untimed launch."""
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=device)
    stream = _stream(torch.device(device))
    flops = blocks * 16 * iters * 32768        # four waves, four products per iteration each

    def launch():
        st = library().sla_diag_mfma_rate(_ptr(sink), blocks, iters, stream)
        if st != 0:
            raise SlaError(st, "sla_diag_mfma_rate")
    launch()
    times = []
    for _ in range(repeats):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        launch()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) * 1e-3)
    times.sort()
    return flops / times[len(times) // 2] / 1e12


# ----------------------------------------------------------------------------- Taylor router
def sla_route_taylor(q, k, top_k: int, block: int = 64,
                     workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Training-free router: int32 block indices [B, H, ceil(n_q/block), top_k]."""
    p = make_problem(q, k, top_k, block)
    _check(q, k, buffers=(workspace,))
    ws = _workspace(p, VARIANT_FORWARD, q.device, workspace)
    idx = torch.empty((p.batch, p.heads, -(-p.n_q // block), top_k), dtype=torch.int32,
                      device=q.device)
    st = library().sla_route_taylor(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(idx), _ptr(ws),
                                    ctypes.c_size_t(_nbytes(ws)), _stream(q.device))
    if st != 0:
        raise SlaError(st, "sla_route_taylor")
    return idx


def sla_forward_taylor(q, k, v, alpha, top_k: int, block: int = 64,
                       out_dtype: torch.dtype = torch.float32, return_idx: bool = True,
                       workspace: Optional[torch.Tensor] = None,
                       out: Optional[torch.Tensor] = None):
    """SLA2 forward with the training-free router. Returns (O, block_idx or None)."""
    p = make_problem(q, k, top_k, block, out_dtype)
    _check(q, k, v, alpha=alpha, out=out, out_dtype=out_dtype, buffers=(workspace,))
    ws = _workspace(p, VARIANT_TAYLOR, q.device, workspace)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    idx = None
    if return_idx:
        idx = torch.empty((p.batch, p.heads, -(-p.n_q // block), top_k), dtype=torch.int32,
                          device=q.device)
    st = library().sla_forward_taylor(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                      _ptr(out), _ptr(idx), _ptr(ws), ctypes.c_size_t(_nbytes(ws)),
                                      _stream(q.device))
    if st != 0:
        raise SlaError(st, "sla_forward_taylor")
    return out, idx


def sla_forward_pisa(q, k, v, proj_q, proj_k, top_k: int, block: int = 64,
                     out_dtype: torch.dtype = torch.float32, return_idx: bool = True,
                     workspace: Optional[torch.Tensor] = None,
                     out: Optional[torch.Tensor] = None):
    """Piecewise exact-or-approximate forward (learnable router; exact routed blocks, Taylor
    tail for the rest, one normalisation). Returns (O, block_idx or None)."""
    p = make_problem(q, k, top_k, block, out_dtype)
    _check(q, k, v, (proj_q, proj_k), out=out, out_dtype=out_dtype, buffers=(workspace,))
    ws = _workspace(p, VARIANT_PISA, q.device, workspace)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    idx = None
    if return_idx:
        idx = torch.empty((p.batch, p.heads, -(-p.n_q // block), top_k), dtype=torch.int32,
                          device=q.device)
    st = library().sla_forward_pisa(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(proj_q),
                                    _ptr(proj_k), _ptr(out), _ptr(idx), _ptr(ws),
                                    ctypes.c_size_t(_nbytes(ws)), _stream(q.device))
    if st != 0:
        raise SlaError(st, "sla_forward_pisa")
    return out, idx
