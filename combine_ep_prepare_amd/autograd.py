"""Autograd-aware dispatch and combine on top of the C ABI.

The PyTorch page of the pages ("[PyTorch] Expert Parallelism: PyTorch
wrapper + autograd ops with symm-mem zero-copy", section "Public Python API")
exposes dispatch and combine as differentiable ops with a per-call routing
state (one per in-flight microbatch). This module does the same for the
one-GPU library: `EpRouting` holds the layout and the handle of one prepared
routing, `dispatch` and `combine` are `torch.autograd.Function`s whose
backward passes call `ep_dispatch_bwd` and `ep_combine_bwd`. Given the
received weights, `combine` applies them itself (the fused weighted combine,
made optional in the same page's review thread on the weight multiply); its
backward calls `ep_combine_weighted_bwd` for both the rows' and the weights'
gradients.

Outputs are allocated with PyTorch; every step of the computation runs in the
library's kernels. A gradient that does not flow into the received weights
arrives here as None and is passed to the library as NULL (the weight
gradient is then zero), the case the pages' review flagged (section
"Greptile Summary").

Every expert-major buffer these ops allocate is defined in full: rows at or
past the live total (``routing.expert_offsets[E]``) of the receive buffer,
of its weights and of the gradients passed back by ``combine`` are zeros
(the library's tail policy, LAYOUT_ZERO_TAIL; combine never reads those rows,
so zero is their exact gradient), and so are pad rows below the total. An
expert function applied to the whole buffer (a parameter shared by every
row, a reduction over it) therefore gets exact parameter gradients. With
``EpRouting(..., zero_tail=False)`` the tail is left unwritten (one zero
write per tail row saved) and such a function must slice the buffer to its
live rows first; with ``fill_pads=False`` pad rows are unwritten too.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import (Layout, combine as _combine, combine_bwd as _combine_bwd,
               combine_weighted as _combine_weighted,
               combine_weighted_bwd as _combine_weighted_bwd, dispatch as _dispatch,
               dispatch_bwd as _dispatch_bwd, new_handle, prepare, recv_capacity_worst)


class EpRouting:
    """One prepared routing: handle, token counts and segment offsets. The
    handle does not depend on the payload type, so one routing serves bf16,
    fp16 and fp32 payloads; ``fill_pads=False`` leaves pad rows unwritten;
    ``zero_tail=False`` leaves the rows past the live total unwritten."""

    def __init__(self, topk_idx: torch.Tensor, num_experts: int, alignment: int, hidden: int,
                 recv_capacity: Optional[int] = None, fill_pads: bool = True,
                 zero_tail: bool = True):
        if topk_idx.dtype != torch.int64:
            raise TypeError("topk_idx must be int64")
        T, K = topk_idx.shape
        if recv_capacity is None:
            recv_capacity = recv_capacity_worst(T, K, num_experts, alignment)
        self._dims = (T, K, num_experts, alignment, hidden, recv_capacity)
        self.fill_pads = fill_pads
        self.zero_tail = zero_tail
        self._layouts = {}
        self.layout = self.layout_for(torch.bfloat16)
        self.handle = new_handle(self.layout, device=topk_idx.device)
        self.token_counts = torch.empty(num_experts, dtype=torch.int32, device=topk_idx.device)
        self.expert_offsets = torch.empty(num_experts + 1, dtype=torch.int32,
                                          device=topk_idx.device)
        prepare(self.layout, topk_idx.contiguous(), self.token_counts, self.handle,
                self.expert_offsets)

    def layout_for(self, dtype: torch.dtype) -> Layout:
        """The layout of this routing for payloads of ``dtype``."""
        if dtype not in self._layouts:
            self._layouts[dtype] = Layout(*self._dims, dtype=dtype, fill_pads=self.fill_pads,
                                          zero_tail=self.zero_tail)
        return self._layouts[dtype]


class _Dispatch(torch.autograd.Function):
    @staticmethod
    def forward(ctx, tokens, topk_weights, routing: EpRouting):
        L = routing.layout_for(tokens.dtype)
        recv = torch.empty(L.cap, L.H, dtype=tokens.dtype, device=tokens.device)
        recv_w = torch.empty(L.cap, dtype=torch.float32, device=tokens.device)
        _dispatch(L, routing.handle, tokens.contiguous(), topk_weights.contiguous(), recv,
                  recv_w)
        ctx.routing = routing
        ctx.dtype = tokens.dtype
        ctx.set_materialize_grads(False)      # an unused output's gradient stays None
        return recv, recv_w

    @staticmethod
    def backward(ctx, g_recv, g_recv_w):
        routing = ctx.routing
        L = routing.layout_for(ctx.dtype)
        grad_tokens = None
        grad_w = None
        want_tokens, want_w = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        if want_tokens or want_w:
            if g_recv is None:
                g_recv = torch.zeros(L.cap, L.H, dtype=ctx.dtype, device=routing.handle.device)
            grad_tokens = torch.empty(L.T, L.H, dtype=g_recv.dtype, device=g_recv.device)
            grad_w = torch.empty(L.T, L.K, dtype=torch.float32, device=g_recv.device)
            _dispatch_bwd(L, routing.handle, g_recv.contiguous(),
                          None if g_recv_w is None else g_recv_w.contiguous(), grad_tokens,
                          grad_w)
        return (grad_tokens if want_tokens else None, grad_w if want_w else None, None)


class _Combine(torch.autograd.Function):
    @staticmethod
    def forward(ctx, expert_out, routing: EpRouting):
        L = routing.layout_for(expert_out.dtype)
        result = torch.empty(L.T, L.H, dtype=expert_out.dtype, device=expert_out.device)
        _combine(L, routing.handle, expert_out.contiguous(), result)
        ctx.routing = routing
        return result

    @staticmethod
    def backward(ctx, g_result):
        routing = ctx.routing
        L = routing.layout_for(g_result.dtype)
        grad = torch.empty(L.cap, L.H, dtype=g_result.dtype, device=g_result.device)
        _combine_bwd(L, routing.handle, g_result.contiguous(), grad)
        return grad, None


class _CombineWeighted(torch.autograd.Function):
    @staticmethod
    def forward(ctx, expert_out, recv_topk_weights, routing: EpRouting):
        L = routing.layout_for(expert_out.dtype)
        expert_out = expert_out.contiguous()
        recv_topk_weights = recv_topk_weights.contiguous()
        result = torch.empty(L.T, L.H, dtype=expert_out.dtype, device=expert_out.device)
        _combine_weighted(L, routing.handle, expert_out, recv_topk_weights, result)
        ctx.routing = routing
        ctx.save_for_backward(expert_out, recv_topk_weights)
        return result

    @staticmethod
    def backward(ctx, g_result):
        expert_out, recv_topk_weights = ctx.saved_tensors
        routing = ctx.routing
        L = routing.layout_for(expert_out.dtype)
        want_rows, want_w = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        if not (want_rows or want_w):
            return None, None, None
        grad_rows = torch.empty(L.cap, L.H, dtype=g_result.dtype, device=g_result.device)
        grad_w = (torch.empty(L.cap, dtype=torch.float32, device=g_result.device)
                  if want_w else None)
        _combine_weighted_bwd(L, routing.handle, g_result.contiguous(),
                              expert_out if want_w else None, recv_topk_weights, grad_rows,
                              grad_w)
        return grad_rows if want_rows else None, grad_w, None


def dispatch(tokens: torch.Tensor, topk_weights: torch.Tensor, routing: EpRouting):
    """(recv_tokens [cap,H], recv_topk_weights [cap]); rows past the live total
    are zeros (unless the routing was made with ``zero_tail=False``)."""
    return _Dispatch.apply(tokens, topk_weights, routing)


def combine(expert_out: torch.Tensor, routing: EpRouting,
            recv_topk_weights: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Sum of each token's expert rows, [T,H]: unweighted, or, given the
    received weights, each row scaled by its route's weight inside the sum."""
    if recv_topk_weights is None:
        return _Combine.apply(expert_out, routing)
    return _CombineWeighted.apply(expert_out, recv_topk_weights, routing)
