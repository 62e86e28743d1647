"""The routing ops as ``torch.library`` custom ops, with autograd and fake
(meta) implementations, so that they can sit inside a ``torch.compile``
graph and be captured in a CUDA/HIP graph.

"[PyTorch] Expert Parallelism: PyTorch wrapper + autograd ops with symm-mem
zero-copy" (sections "Summary" and "Public Python API") registers dispatch and
combine as ``torch.library.custom_op`` with ``mutates_args`` and autograd
support; this module does the same for the one-GPU library. Every op
allocates its outputs with PyTorch and calls the C entry point of the same
name; nothing is computed here.

A layout travels as a list of ints ``[T, K, E, A, H, recv_capacity, dtype,
flags]`` (``layout_list``); the handle is the uint8 device tensor that
``prepare`` fills (declared mutated by prepare, read by the others).
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import torch
from torch import Tensor

from . import (DTYPE_BF16, LAYOUT_NO_PAD_FILL, LAYOUT_ZERO_TAIL, TORCH_DTYPE, Layout,
               combine as _combine,
               combine_bwd as _combine_bwd, combine_weighted as _combine_weighted,
               combine_weighted_bwd as _combine_weighted_bwd, dispatch as _dispatch,
               dispatch_bwd as _dispatch_bwd, prepare as _prepare)

NS = "ep_mi355x"


def layout_list(layout: Layout) -> List[int]:
    return [int(layout.num_tokens), int(layout.topk), int(layout.num_experts),
            int(layout.alignment), int(layout.hidden), int(layout.recv_capacity),
            int(layout.dtype), int(layout.flags)]


def _layout(ll: Sequence[int], zero_tail: bool = False) -> Layout:
    """The layout of a list; ``zero_tail`` adds LAYOUT_ZERO_TAIL, which every
    op below that allocates an expert-major output sets, so that its rows past
    the live total are zeros rather than uninitialised memory."""
    T, K, E, A, H, cap, dt, flags = ll
    return Layout(T, K, E, A, H, cap, dtype=dt, fill_pads=not (flags & LAYOUT_NO_PAD_FILL),
                  zero_tail=zero_tail or bool(flags & LAYOUT_ZERO_TAIL))


def _pdtype(ll: Sequence[int]) -> torch.dtype:
    return TORCH_DTYPE.get(ll[6], TORCH_DTYPE[DTYPE_BF16])


# --------------------------------------------------------------------------
# prepare
# --------------------------------------------------------------------------

@torch.library.custom_op(f"{NS}::prepare", mutates_args=("handle",))
def prepare(topk_idx: Tensor, handle: Tensor, layout: List[int]) -> Tuple[Tensor, Tensor]:
    """(token_counts int32 [E], expert_offsets int32 [E+1]); fills ``handle``."""
    L = _layout(layout)
    counts = torch.empty(L.E, dtype=torch.int32, device=topk_idx.device)
    offsets = torch.empty(L.E + 1, dtype=torch.int32, device=topk_idx.device)
    _prepare(L, topk_idx, counts, handle, offsets)
    return counts, offsets


@prepare.register_fake
def _(topk_idx, handle, layout):
    E = layout[2]
    return (topk_idx.new_empty((E,), dtype=torch.int32),
            topk_idx.new_empty((E + 1,), dtype=torch.int32))


# --------------------------------------------------------------------------
# dispatch and its backward
# --------------------------------------------------------------------------

@torch.library.custom_op(f"{NS}::dispatch", mutates_args=())
def dispatch(tokens: Tensor, topk_weights: Tensor, handle: Tensor,
             layout: List[int]) -> Tuple[Tensor, Tensor]:
    """(recv_tokens [cap,H], recv_topk_weights fp32 [cap]); rows past the live
    total are zeros."""
    L = _layout(layout, zero_tail=True)
    recv = torch.empty(L.cap, L.H, dtype=tokens.dtype, device=tokens.device)
    recv_w = torch.empty(L.cap, dtype=torch.float32, device=tokens.device)
    _dispatch(L, handle, tokens, topk_weights, recv, recv_w)
    return recv, recv_w


@dispatch.register_fake
def _(tokens, topk_weights, handle, layout):
    cap, H = layout[5], layout[4]
    return tokens.new_empty((cap, H)), tokens.new_empty((cap,), dtype=torch.float32)


@torch.library.custom_op(f"{NS}::dispatch_bwd", mutates_args=())
def dispatch_bwd(grad: Tensor, g_recv_topk_weights: Optional[Tensor], handle: Tensor,
                 layout: List[int]) -> Tuple[Tensor, Tensor]:
    """(grad_tokens [T,H], grad_topk_weights fp32 [T,K]); a None weight
    gradient gives zero weight gradients."""
    L = _layout(layout)
    gt = torch.empty(L.T, L.H, dtype=grad.dtype, device=grad.device)
    gw = torch.empty(L.T, L.K, dtype=torch.float32, device=grad.device)
    _dispatch_bwd(L, handle, grad, g_recv_topk_weights, gt, gw)
    return gt, gw


@dispatch_bwd.register_fake
def _(grad, g_recv_topk_weights, handle, layout):
    T, K, H = layout[0], layout[1], layout[4]
    return grad.new_empty((T, H)), grad.new_empty((T, K), dtype=torch.float32)


def _dispatch_setup(ctx, inputs, output):
    _, _, handle, layout = inputs
    ctx.save_for_backward(handle)
    ctx.layout = layout


def _dispatch_backward(ctx, g_recv, g_recv_w):
    (handle,) = ctx.saved_tensors
    layout = ctx.layout
    if g_recv is None:
        g_recv = torch.zeros(layout[5], layout[4], dtype=_pdtype(layout), device=handle.device)
    gt, gw = dispatch_bwd(g_recv.contiguous(),
                          None if g_recv_w is None else g_recv_w.contiguous(), handle, layout)
    return gt, gw, None, None


dispatch.register_autograd(_dispatch_backward, setup_context=_dispatch_setup)


# --------------------------------------------------------------------------
# combine and its backward
# --------------------------------------------------------------------------

@torch.library.custom_op(f"{NS}::combine", mutates_args=())
def combine(expert_out: Tensor, handle: Tensor, layout: List[int]) -> Tensor:
    """Unweighted sum of each token's received rows, [T,H]."""
    L = _layout(layout)
    out = torch.empty(L.T, L.H, dtype=expert_out.dtype, device=expert_out.device)
    _combine(L, handle, expert_out, out)
    return out


@combine.register_fake
def _(expert_out, handle, layout):
    return expert_out.new_empty((layout[0], layout[4]))


@torch.library.custom_op(f"{NS}::combine_bwd", mutates_args=())
def combine_bwd(grad: Tensor, handle: Tensor, layout: List[int]) -> Tensor:
    """grad_expert_out [cap,H]: each live row takes its token's gradient; pad
    rows zero (unless the layout skips the pad fill); rows past the live total
    zero (combine never reads them)."""
    L = _layout(layout, zero_tail=True)
    out = torch.empty(L.cap, L.H, dtype=grad.dtype, device=grad.device)
    _combine_bwd(L, handle, grad, out)
    return out


@combine_bwd.register_fake
def _(grad, handle, layout):
    return grad.new_empty((layout[5], layout[4]))


def _combine_setup(ctx, inputs, output):
    _, handle, layout = inputs
    ctx.save_for_backward(handle)
    ctx.layout = layout


def _combine_backward(ctx, g):
    (handle,) = ctx.saved_tensors
    return combine_bwd(g.contiguous(), handle, ctx.layout), None, None


combine.register_autograd(_combine_backward, setup_context=_combine_setup)


# --------------------------------------------------------------------------
# weighted combine and its backward
# --------------------------------------------------------------------------

@torch.library.custom_op(f"{NS}::combine_weighted", mutates_args=())
def combine_weighted(expert_out: Tensor, recv_topk_weights: Tensor, handle: Tensor,
                     layout: List[int]) -> Tensor:
    """Sum of each token's received rows, each scaled by its received weight."""
    L = _layout(layout)
    out = torch.empty(L.T, L.H, dtype=expert_out.dtype, device=expert_out.device)
    _combine_weighted(L, handle, expert_out, recv_topk_weights, out)
    return out


@combine_weighted.register_fake
def _(expert_out, recv_topk_weights, handle, layout):
    return expert_out.new_empty((layout[0], layout[4]))


@torch.library.custom_op(f"{NS}::combine_weighted_bwd", mutates_args=())
def combine_weighted_bwd(grad: Tensor, expert_out: Tensor, recv_topk_weights: Tensor,
                         handle: Tensor, layout: List[int]) -> Tuple[Tensor, Tensor]:
    """(grad_expert_out [cap,H], grad_recv_topk_weights fp32 [cap]); rows past
    the live total zero in both."""
    L = _layout(layout, zero_tail=True)
    gr = torch.empty(L.cap, L.H, dtype=grad.dtype, device=grad.device)
    gw = torch.empty(L.cap, dtype=torch.float32, device=grad.device)
    _combine_weighted_bwd(L, handle, grad, expert_out, recv_topk_weights, gr, gw)
    return gr, gw


@combine_weighted_bwd.register_fake
def _(grad, expert_out, recv_topk_weights, handle, layout):
    cap, H = layout[5], layout[4]
    return grad.new_empty((cap, H)), grad.new_empty((cap,), dtype=torch.float32)


def _cw_setup(ctx, inputs, output):
    expert_out, recv_topk_weights, handle, layout = inputs
    ctx.save_for_backward(expert_out, recv_topk_weights, handle)
    ctx.layout = layout


def _cw_backward(ctx, g):
    expert_out, w, handle = ctx.saved_tensors
    gr, gw = combine_weighted_bwd(g.contiguous(), expert_out, w, handle, ctx.layout)
    return gr, gw, None, None


combine_weighted.register_autograd(_cw_backward, setup_context=_cw_setup)
