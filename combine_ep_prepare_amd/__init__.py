"""Python binding of the MI355X expert-parallel routing library (include/ep.h).

Argument marshalling only: each function checks dtypes, devices, shapes and
contiguity of PyTorch tensors, then calls the C entry point of the same name
in ``libcombine_ep_prepare_amd.so`` with raw device pointers and the current
HIP stream. Every step of the computation runs in the library's kernels.
There is no fallback: if the library is missing, importing the binding
raises.

The five ops follow the per-step calls of "Expert Parallelism: common C API
+ NCCL EP backend" (section "Per-step (allocation-free, CUDA-graph
capturable)"): prepare, dispatch, combine, dispatch_bwd and combine_bwd.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcombine_ep_prepare_amd.so")

EP_OK = 0
EP_ERR_NULL = 1
EP_ERR_SHAPE = 2
EP_ERR_ALIGN = 3
EP_ERR_HANDLE_SIZE = 4
EP_ERR_CAPACITY = 5
EP_ERR_DEVICE = 6
EP_ERR_HIP = 7
EP_ERR_SCRATCH = 8
PREPARE_STATIC_SCRATCH_BYTES = 4 << 20

STATUS_BAD_EXPERT = 1
STATUS_OVERFLOW = 2
STATUS_LAYOUT = 4

DTYPE_BF16 = 0
DTYPE_FP16 = 1
DTYPE_FP32 = 2
LAYOUT_NO_PAD_FILL = 1
LAYOUT_ZERO_TAIL = 4

# payload type code -> torch dtype of the rows
TORCH_DTYPE = {DTYPE_BF16: torch.bfloat16, DTYPE_FP16: torch.float16,
               DTYPE_FP32: torch.float32}
_CODE_OF = {torch.bfloat16: DTYPE_BF16, torch.float16: DTYPE_FP16, torch.float32: DTYPE_FP32,
            "bf16": DTYPE_BF16, "fp16": DTYPE_FP16, "fp32": DTYPE_FP32}

ENTRY_POINTS = ("ep_recv_capacity_worst", "ep_handle_mem_size", "ep_handle_regions",
                "ep_prepare", "ep_prepare_static", "ep_dispatch",
                "ep_combine", "ep_dispatch_bwd", "ep_combine_bwd", "ep_combine_weighted",
                "ep_combine_weighted_bwd", "ep_read_status", "ep_status_str")


class Layout(C.Structure):
    """ep_layout_t. ``dtype`` is the payload type (a torch dtype, "bf16",
    "fp16", "fp32" or a DTYPE_* code); ``fill_pads=False`` sets
    LAYOUT_NO_PAD_FILL; ``zero_tail=True`` sets LAYOUT_ZERO_TAIL
    (expert-major outputs also get zeros in the rows past the live total)."""
    _fields_ = [("num_tokens", C.c_int64), ("topk", C.c_int32), ("num_experts", C.c_int32),
                ("alignment", C.c_int32), ("dtype", C.c_uint16), ("flags", C.c_uint16),
                ("hidden", C.c_int64), ("recv_capacity", C.c_int64)]

    def __init__(self, num_tokens, topk, num_experts, alignment, hidden, recv_capacity,
                 dtype=DTYPE_BF16, fill_pads=True, zero_tail=False):
        code = dtype if isinstance(dtype, int) else _CODE_OF[dtype]
        flags = (0 if fill_pads else LAYOUT_NO_PAD_FILL) | (LAYOUT_ZERO_TAIL if zero_tail else 0)
        super().__init__(num_tokens, topk, num_experts, alignment, code, flags, hidden,
                         recv_capacity)

    @property
    def payload_dtype(self) -> torch.dtype:
        """torch dtype of the payload rows (bfloat16 for an unknown code)."""
        return TORCH_DTYPE.get(self.dtype, torch.bfloat16)

    @property
    def T(self):
        return self.num_tokens

    @property
    def K(self):
        return self.topk

    @property
    def E(self):
        return self.num_experts

    @property
    def A(self):
        return self.alignment

    @property
    def H(self):
        return self.hidden

    @property
    def cap(self):
        return self.recv_capacity


class HandleRegions(C.Structure):
    """ep_handle_regions_t: byte offsets of the routing maps in a handle."""
    _fields_ = [("status", C.c_size_t), ("counts", C.c_size_t), ("offsets", C.c_size_t),
                ("slot", C.c_size_t), ("row_src", C.c_size_t), ("bytes", C.c_size_t),
                ("runs", C.c_size_t), ("maps_bytes", C.c_size_t),
                ("stream_live", C.c_size_t), ("run_units", C.c_size_t),
                ("run_list_entries", C.c_size_t)]


class EpError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {status_str(code)} (ep_status_t {code})")
        self.code = code


def _load_library(path: str = LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; "
            "g.build()'` (hipcc, gfx950)")
    lib = C.CDLL(path)
    i64, i32, vp, sz = C.c_int64, C.c_int32, C.c_void_p, C.c_size_t
    lp = C.POINTER(Layout)
    lib.ep_recv_capacity_worst.argtypes = [i64, i32, i32, i32]
    lib.ep_recv_capacity_worst.restype = i64
    lib.ep_handle_mem_size.argtypes = [lp]
    lib.ep_handle_mem_size.restype = sz
    lib.ep_handle_regions.argtypes = [lp, C.POINTER(HandleRegions)]
    lib.ep_handle_regions.restype = C.c_int
    lib.ep_prepare.argtypes = [lp, vp, vp, vp, vp, sz, vp]
    lib.ep_prepare_static.argtypes = [lp, vp, vp, vp, vp, sz, vp]
    lib.ep_dispatch.argtypes = [lp, vp, sz, vp, vp, vp, vp, vp]
    lib.ep_combine.argtypes = [lp, vp, sz, vp, vp, vp]
    lib.ep_dispatch_bwd.argtypes = [lp, vp, sz, vp, vp, vp, vp, vp]
    lib.ep_combine_bwd.argtypes = [lp, vp, sz, vp, vp, vp]
    lib.ep_combine_weighted.argtypes = [lp, vp, sz, vp, vp, vp, vp]
    lib.ep_combine_weighted_bwd.argtypes = [lp, vp, sz, vp, vp, vp, vp, vp, vp]
    lib.ep_read_status.argtypes = [vp, C.POINTER(C.c_uint32), vp]
    for name in ("ep_prepare", "ep_prepare_static", "ep_dispatch", "ep_combine",
                 "ep_dispatch_bwd",
                 "ep_combine_bwd", "ep_combine_weighted", "ep_combine_weighted_bwd",
                 "ep_read_status"):
        getattr(lib, name).restype = C.c_int
    lib.ep_status_str.argtypes = [C.c_int]
    lib.ep_status_str.restype = C.c_char_p
    return lib


lib = _load_library()


def status_str(code: int) -> str:
    return lib.ep_status_str(code).decode()


def _check(code: int, what: str):
    if code != EP_OK:
        raise EpError(code, what)


def recv_capacity_worst(T: int, K: int, E: int, A: int) -> int:
    return int(lib.ep_recv_capacity_worst(T, K, E, A))


def handle_mem_size(layout: Layout) -> int:
    return int(lib.ep_handle_mem_size(C.byref(layout)))


def handle_regions(layout: Layout) -> HandleRegions:
    out = HandleRegions()
    _check(lib.ep_handle_regions(C.byref(layout), C.byref(out)), "ep_handle_regions")
    return out


def handle_maps(layout: Layout, handle: torch.Tensor) -> dict:
    """Views of the routing maps inside a prepared handle (no copy)."""
    r = handle_regions(layout)

    def view(off, n, dtype):
        return handle[off:off + 4 * n].view(dtype)

    return {
        "status": view(r.status, 1, torch.int32),
        "counts": view(r.counts, layout.E, torch.int32),
        "offsets": view(r.offsets, layout.E + 1, torch.int32),
        "slot": view(r.slot, layout.T * layout.K, torch.int32),
        "row_src": view(r.row_src, layout.cap, torch.int32),
        "runs": view(r.runs, 8 * 2 * r.run_list_entries, torch.int32).view(8, -1, 2),
        "stream_live": view(r.stream_live, 8, torch.int32),
        "run_units": view(r.run_units, 1, torch.int32),
    }


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream) -> C.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _need(t: Optional[torch.Tensor], name: str, dtype, shape=None, allow_none=False):
    if t is None:
        if allow_none:
            return
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}; the library runs on the current device "
                         f"cuda:{torch.cuda.current_device()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def new_handle(layout: Layout, device=None) -> torch.Tensor:
    """Allocate the caller-owned handle memory for ``layout`` (uint8 tensor)."""
    n = handle_mem_size(layout)
    if n == 0:
        raise ValueError("invalid layout")
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def prepare(layout: Layout, topk_idx: torch.Tensor, token_counts: torch.Tensor,
            handle: torch.Tensor, expert_offsets: Optional[torch.Tensor] = None,
            stream=None):
    _need(topk_idx, "topk_idx", torch.int64, (layout.T, layout.K))
    _need(token_counts, "token_counts", torch.int32, (layout.E,))
    _need(expert_offsets, "expert_offsets", torch.int32, (layout.E + 1,), allow_none=True)
    _need(handle, "handle", torch.uint8)
    _check(lib.ep_prepare(C.byref(layout), _ptr(topk_idx), _ptr(token_counts),
                          _ptr(expert_offsets), _ptr(handle), handle.numel(),
                          _stream(stream)), "ep_prepare")


def prepare_static(layout: Layout, topk_idx: torch.Tensor, token_counts: torch.Tensor,
                   handle: torch.Tensor, expert_offsets: Optional[torch.Tensor] = None,
                   stream=None):
    """prepare with its scratch in the library's static device array: the
    handle needs only ``handle_regions(layout).maps_bytes`` bytes. Calls that
    overlap on one device race."""
    _need(topk_idx, "topk_idx", torch.int64, (layout.T, layout.K))
    _need(token_counts, "token_counts", torch.int32, (layout.E,))
    _need(expert_offsets, "expert_offsets", torch.int32, (layout.E + 1,), allow_none=True)
    _need(handle, "handle", torch.uint8)
    _check(lib.ep_prepare_static(C.byref(layout), _ptr(topk_idx), _ptr(token_counts),
                                 _ptr(expert_offsets), _ptr(handle), handle.numel(),
                                 _stream(stream)), "ep_prepare_static")


def dispatch(layout: Layout, handle: torch.Tensor, tokens: torch.Tensor,
             topk_weights: Optional[torch.Tensor], recv_tokens: torch.Tensor,
             recv_topk_weights: Optional[torch.Tensor] = None, stream=None):
    _need(handle, "handle", torch.uint8)
    _need(tokens, "tokens", layout.payload_dtype, (layout.T, layout.H))
    _need(topk_weights, "topk_weights", torch.float32, (layout.T, layout.K), allow_none=True)
    _need(recv_tokens, "recv_tokens", layout.payload_dtype, (layout.cap, layout.H))
    _need(recv_topk_weights, "recv_topk_weights", torch.float32, (layout.cap,),
          allow_none=True)
    _check(lib.ep_dispatch(C.byref(layout), _ptr(handle), handle.numel(), _ptr(tokens),
                           _ptr(topk_weights), _ptr(recv_tokens), _ptr(recv_topk_weights),
                           _stream(stream)), "ep_dispatch")


def combine(layout: Layout, handle: torch.Tensor, expert_out: torch.Tensor,
            result: torch.Tensor, stream=None):
    _need(handle, "handle", torch.uint8)
    _need(expert_out, "expert_out", layout.payload_dtype, (layout.cap, layout.H))
    _need(result, "result", layout.payload_dtype, (layout.T, layout.H))
    _check(lib.ep_combine(C.byref(layout), _ptr(handle), handle.numel(), _ptr(expert_out),
                          _ptr(result), _stream(stream)), "ep_combine")


def dispatch_bwd(layout: Layout, handle: torch.Tensor, grad: torch.Tensor,
                 g_recv_topk_weights: Optional[torch.Tensor], grad_tokens: torch.Tensor,
                 grad_topk_weights: Optional[torch.Tensor] = None, stream=None):
    _need(handle, "handle", torch.uint8)
    _need(grad, "grad", layout.payload_dtype, (layout.cap, layout.H))
    _need(g_recv_topk_weights, "g_recv_topk_weights", torch.float32, (layout.cap,),
          allow_none=True)
    _need(grad_tokens, "grad_tokens", layout.payload_dtype, (layout.T, layout.H))
    _need(grad_topk_weights, "grad_topk_weights", torch.float32, (layout.T, layout.K),
          allow_none=True)
    _check(lib.ep_dispatch_bwd(C.byref(layout), _ptr(handle), handle.numel(), _ptr(grad),
                               _ptr(g_recv_topk_weights), _ptr(grad_tokens),
                               _ptr(grad_topk_weights), _stream(stream)), "ep_dispatch_bwd")


def combine_bwd(layout: Layout, handle: torch.Tensor, grad: torch.Tensor,
                grad_expert_out: torch.Tensor, stream=None):
    _need(handle, "handle", torch.uint8)
    _need(grad, "grad", layout.payload_dtype, (layout.T, layout.H))
    _need(grad_expert_out, "grad_expert_out", layout.payload_dtype, (layout.cap, layout.H))
    _check(lib.ep_combine_bwd(C.byref(layout), _ptr(handle), handle.numel(), _ptr(grad),
                              _ptr(grad_expert_out), _stream(stream)), "ep_combine_bwd")


def combine_weighted(layout: Layout, handle: torch.Tensor, expert_out: torch.Tensor,
                     recv_topk_weights: torch.Tensor, result: torch.Tensor, stream=None):
    _need(handle, "handle", torch.uint8)
    _need(expert_out, "expert_out", layout.payload_dtype, (layout.cap, layout.H))
    _need(recv_topk_weights, "recv_topk_weights", torch.float32, (layout.cap,))
    _need(result, "result", layout.payload_dtype, (layout.T, layout.H))
    _check(lib.ep_combine_weighted(C.byref(layout), _ptr(handle), handle.numel(),
                                   _ptr(expert_out), _ptr(recv_topk_weights), _ptr(result),
                                   _stream(stream)), "ep_combine_weighted")


def combine_weighted_bwd(layout: Layout, handle: torch.Tensor, grad: torch.Tensor,
                         expert_out: Optional[torch.Tensor], recv_topk_weights: torch.Tensor,
                         grad_expert_out: torch.Tensor,
                         grad_recv_topk_weights: Optional[torch.Tensor] = None, stream=None):
    _need(handle, "handle", torch.uint8)
    _need(grad, "grad", layout.payload_dtype, (layout.T, layout.H))
    _need(expert_out, "expert_out", layout.payload_dtype, (layout.cap, layout.H), allow_none=True)
    _need(recv_topk_weights, "recv_topk_weights", torch.float32, (layout.cap,))
    _need(grad_expert_out, "grad_expert_out", layout.payload_dtype, (layout.cap, layout.H))
    _need(grad_recv_topk_weights, "grad_recv_topk_weights", torch.float32, (layout.cap,),
          allow_none=True)
    _check(lib.ep_combine_weighted_bwd(C.byref(layout), _ptr(handle), handle.numel(),
                                       _ptr(grad), _ptr(expert_out), _ptr(recv_topk_weights),
                                       _ptr(grad_expert_out), _ptr(grad_recv_topk_weights),
                                       _stream(stream)), "ep_combine_weighted_bwd")


def read_status(handle: torch.Tensor, stream=None) -> int:
    """Status word of the handle (waits for the stream)."""
    _need(handle, "handle", torch.uint8)
    out = C.c_uint32(0)
    _check(lib.ep_read_status(_ptr(handle), C.byref(out), _stream(stream)), "ep_read_status")
    return int(out.value)
