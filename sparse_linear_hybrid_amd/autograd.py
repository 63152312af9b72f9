"""torch.autograd wrapper around sla_forward / sla_backward (argument marshalling only).

``sla_attention(q, k, v, proj_q, proj_k, alpha, top_k)`` returns O (fp32) and, when any of
q, k, v, alpha requires grad, records the forward's block selection so that backward calls
``sla_backward`` at that selection. The router's top-k is piecewise constant, so proj_q and
proj_k receive no gradient (None); q, k, v, alpha get the gradients of the forward at the
fixed selection (SLA2 page, section 2.B: training differentiates through a relaxed top-k the
page does not define; section 2.C: with ``fp8=True`` the forward runs the quantised sparse
branch and the gradients are the unquantised branch's, the straight-through reading).
"""
from __future__ import annotations

import torch

from . import sla as _sla


class SLAAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, proj_q, proj_k, alpha, top_k: int, block: int, fp8: bool):
        fwd = _sla.sla_forward_fp8 if fp8 else _sla.sla_forward
        out, idx = fwd(q, k, v, proj_q, proj_k, alpha, top_k, block=block,
                       out_dtype=torch.float32)
        ctx.save_for_backward(q, k, v, alpha, idx)
        ctx.block = block
        ctx.mark_non_differentiable(idx)
        return out, idx

    @staticmethod
    def backward(ctx, dout, _didx):
        q, k, v, alpha, idx = ctx.saved_tensors
        if dout is None:
            return (None,) * 9
        dq, dk, dv, dal = _sla.sla_backward(q, k, v, alpha, dout.contiguous().float(), idx,
                                            block=ctx.block)
        cast = lambda g, like: g.to(like.dtype) if g.dtype != like.dtype else g   # noqa: E731
        return (cast(dq, q), cast(dk, k), cast(dv, v), None, None, cast(dal, alpha),
                None, None, None)


def sla_attention(q, k, v, proj_q, proj_k, alpha, top_k: int, block: int = 64,
                  fp8: bool = False, return_idx: bool = False):
    """SLA2 forward (fp32 output) with autograd support for q, k, v and alpha (bf16 inputs
    for the backward). Returns O, or (O, block_idx) with return_idx."""
    out, idx = SLAAttention.apply(q, k, v, proj_q, proj_k, alpha, top_k, block, fp8)
    return (out, idx) if return_idx else out
