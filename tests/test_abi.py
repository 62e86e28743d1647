"""Host-side checks of the C ABI (no GPU needed).

- the library loads and exports every function include/ep.h declares;
- size queries (handle size, worst-case capacity, handle regions);
- every host-detectable error returns its code before any HIP call. Each
  case below fails validation, so no device pointer is ever dereferenced.
"""
import ctypes as C
import os
import re

import pytest

import combine_ep_prepare_amd as ep

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ep.h")

# Fake, never dereferenced device addresses (16-byte aligned / misaligned).
P = C.c_void_p(0x10000)
P2 = C.c_void_p(0x20000)
MIS = C.c_void_p(0x10008)


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ep_[a-z_]+)\s*\(", text)))


def test_every_declared_function_is_exported():
    names = _declared_functions()
    assert len(names) >= 10
    lib = C.CDLL(ep.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in ep.h but not exported"
    assert set(names) == set(ep.ENTRY_POINTS)


def lay(T=16, K=2, E=4, A=8, H=64, cap=None):
    if cap is None:
        cap = max(64, ep.recv_capacity_worst(T, K, E, A))
    return ep.Layout(T, K, E, A, H, cap)


def test_recv_capacity_worst():
    assert ep.recv_capacity_worst(4096, 8, 256, 128) == 4096 * 8 + 256 * 127
    assert ep.recv_capacity_worst(10, 8, 4, 1) == 40         # K > E: min(K, E) routes
    assert ep.recv_capacity_worst(0, 8, 32, 128) == 32 * 127
    assert ep.recv_capacity_worst(-1, 8, 32, 128) == -1
    assert ep.recv_capacity_worst(1, 0, 32, 128) == -1


def test_handle_size_and_regions():
    L = lay(T=4096, K=8, E=256, A=128, H=7168)
    n = ep.handle_mem_size(L)
    r = ep.handle_regions(L)
    assert r.bytes == n
    for off in (r.counts, r.offsets, r.slot, r.row_src):
        assert off % 256 == 0
    assert r.counts + 4 * 256 <= r.offsets
    assert r.offsets + 4 * 257 <= r.slot
    assert r.slot + 4 * 4096 * 8 <= r.row_src
    assert r.row_src + 4 * L.cap <= n
    assert r.runs % 256 == 0 and r.row_src + 4 * L.cap <= r.runs
    # the run entries close the maps: eight stream lists of 64 U + 2048
    # entries each (U = 64 units of 512 routes), 8 bytes an entry
    assert r.runs + 8 * (64 * 64 + 2048) * 8 == r.maps_bytes
    # prepare's scratch closes the handle: 256-expert histograms of the 64
    # units of 512 routes, of their 16 blocks of 4 units and one totals row,
    # then two words per unit (its flags, a chunk start), each part
    # 256-byte aligned
    assert n - r.maps_bytes == (64 + 16 + 1) * 256 * 4 + 512
    # the handle grows with the capacity and does not depend on H
    assert ep.handle_mem_size(lay(T=4096, K=8, E=256, A=128, H=512)) == n
    assert ep.handle_mem_size(lay(T=4096, K=8, E=256, A=128, H=7168, cap=L.cap * 2)) > n


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), ep.EP_ERR_SHAPE),
    (dict(K=0), ep.EP_ERR_SHAPE),
    (dict(K=65), ep.EP_ERR_SHAPE),
    (dict(E=0), ep.EP_ERR_SHAPE),
    (dict(E=2049), ep.EP_ERR_SHAPE),
    (dict(A=0), ep.EP_ERR_SHAPE),
    (dict(H=0), ep.EP_ERR_SHAPE),
    (dict(H=12), ep.EP_ERR_SHAPE),
    (dict(cap=-1), ep.EP_ERR_CAPACITY),
    (dict(cap=2 ** 31), ep.EP_ERR_CAPACITY),
    (dict(T=2 ** 28, K=8), ep.EP_ERR_SHAPE),           # T*K >= 2^31
    (dict(E=2048, A=2 ** 21, cap=0), ep.EP_ERR_SHAPE),  # E*(A-1) >= 2^31
])
def test_bad_layouts_rejected(kw, code):
    L = lay(**kw)
    assert ep.handle_mem_size(L) == 0
    assert ep.lib.ep_prepare(C.byref(L), P, P, None, P, 1 << 30, None) == code
    assert ep.lib.ep_dispatch(C.byref(L), P, 1 << 30, P, None, P2, None, None) == code
    assert ep.lib.ep_combine(C.byref(L), P, 1 << 30, P, P2, None) == code
    assert ep.lib.ep_dispatch_bwd(C.byref(L), P, 1 << 30, P, None, P2, None, None) == code
    assert ep.lib.ep_combine_bwd(C.byref(L), P, 1 << 30, P, P2, None) == code
    r = ep.HandleRegions()
    assert ep.lib.ep_handle_regions(C.byref(L), C.byref(r)) == code


@pytest.mark.parametrize("dtype,flags,ok", [
    (0, 0, True), (1, 0, True), (2, 0, True), (0, 1, True), (2, 1, True), (0, 4, True),
    (1, 5, True), (3, 0, False), (0xFFFF, 0, False), (0, 2, False), (0, 3, False),
    (2, 7, False), (0, 8, False), (0, 12, False), (0, 0x8001, False),
])
def test_payload_type_and_flags_validated(dtype, flags, ok):
    L = lay()
    L.dtype = dtype
    L.flags = flags
    n = ep.handle_mem_size(L)
    if ok:
        # neither the payload type nor the pad and tail policies change the
        # handle
        assert n == ep.handle_mem_size(lay())
    else:
        assert n == 0
        assert ep.lib.ep_dispatch(C.byref(L), P, 1 << 30, P, None, P2, None, None) == \
            ep.EP_ERR_SHAPE


def test_layout_struct_matches_header():
    # field offsets of ep_layout_t as declared in include/ep.h
    assert C.sizeof(ep.Layout) == 40
    assert [getattr(ep.Layout, f).offset for f in
            ("num_tokens", "topk", "num_experts", "alignment", "dtype", "flags", "hidden",
             "recv_capacity")] == [0, 8, 12, 16, 20, 22, 24, 32]
    L = ep.Layout(4, 2, 8, 16, 512, 100, dtype="fp16", fill_pads=False)
    assert (L.dtype, L.flags) == (ep.DTYPE_FP16, ep.LAYOUT_NO_PAD_FILL)


def test_null_layout_and_pointers():
    L = lay()
    n = ep.handle_mem_size(L)
    assert ep.lib.ep_prepare(None, P, P, None, P, n, None) == ep.EP_ERR_NULL
    assert ep.lib.ep_prepare(C.byref(L), None, P, None, P, n, None) == ep.EP_ERR_NULL
    assert ep.lib.ep_prepare(C.byref(L), P, None, None, P, n, None) == ep.EP_ERR_NULL
    assert ep.lib.ep_prepare(C.byref(L), P, P, None, None, n, None) == ep.EP_ERR_NULL
    assert ep.lib.ep_dispatch(C.byref(L), None, n, P, None, P2, None, None) == ep.EP_ERR_NULL
    assert ep.lib.ep_dispatch(C.byref(L), P, n, None, None, P2, None, None) == ep.EP_ERR_NULL
    assert ep.lib.ep_dispatch(C.byref(L), P, n, P, None, None, None, None) == ep.EP_ERR_NULL
    # weights and received weights must be given together
    assert ep.lib.ep_dispatch(C.byref(L), P, n, P, P2, P2, None, None) == ep.EP_ERR_NULL
    assert ep.lib.ep_dispatch(C.byref(L), P, n, P, None, P2, P2, None) == ep.EP_ERR_NULL
    assert ep.lib.ep_combine(C.byref(L), P, n, None, P2, None) == ep.EP_ERR_NULL
    assert ep.lib.ep_combine(C.byref(L), P, n, P, None, None) == ep.EP_ERR_NULL
    assert ep.lib.ep_dispatch_bwd(C.byref(L), P, n, None, None, P2, None, None) == \
        ep.EP_ERR_NULL
    assert ep.lib.ep_combine_bwd(C.byref(L), P, n, None, P2, None) == ep.EP_ERR_NULL
    assert ep.lib.ep_combine_bwd(C.byref(L), P, n, P, None, None) == ep.EP_ERR_NULL
    out = C.c_uint32(0)
    assert ep.lib.ep_read_status(None, C.byref(out), None) == ep.EP_ERR_NULL
    assert ep.lib.ep_read_status(P, None, None) == ep.EP_ERR_NULL
    assert ep.lib.ep_handle_regions(C.byref(L), None) == ep.EP_ERR_NULL


def test_handle_too_small():
    # prepare needs the whole handle (maps and its scratch); the payload ops
    # read only the maps
    L = lay(T=4096, K=8, E=256, A=128, H=7168)
    n = ep.handle_mem_size(L)
    m = ep.handle_regions(L).maps_bytes
    assert m < n
    assert ep.lib.ep_prepare(C.byref(L), P, P, None, P, n - 1, None) == ep.EP_ERR_HANDLE_SIZE
    assert ep.lib.ep_dispatch(C.byref(L), P, m - 1, P, None, P2, None, None) == \
        ep.EP_ERR_HANDLE_SIZE
    assert ep.lib.ep_combine(C.byref(L), P, 0, P, P2, None) == ep.EP_ERR_HANDLE_SIZE
    assert ep.lib.ep_dispatch_bwd(C.byref(L), P, 7, P, None, P2, None, None) == \
        ep.EP_ERR_HANDLE_SIZE
    assert ep.lib.ep_combine_bwd(C.byref(L), P, m - 256, P, P2, None) == \
        ep.EP_ERR_HANDLE_SIZE


def test_misaligned_pointers():
    L = lay()
    n = ep.handle_mem_size(L)
    assert ep.lib.ep_prepare(C.byref(L), P, P, None, MIS, n, None) == ep.EP_ERR_ALIGN
    assert ep.lib.ep_dispatch(C.byref(L), MIS, n, P, None, P2, None, None) == ep.EP_ERR_ALIGN
    assert ep.lib.ep_dispatch(C.byref(L), P, n, MIS, None, P2, None, None) == ep.EP_ERR_ALIGN
    assert ep.lib.ep_dispatch(C.byref(L), P, n, P, None, MIS, None, None) == ep.EP_ERR_ALIGN
    assert ep.lib.ep_combine(C.byref(L), P, n, MIS, P2, None) == ep.EP_ERR_ALIGN
    assert ep.lib.ep_combine(C.byref(L), P, n, P, MIS, None) == ep.EP_ERR_ALIGN
    assert ep.lib.ep_dispatch_bwd(C.byref(L), P, n, MIS, None, P2, None, None) == \
        ep.EP_ERR_ALIGN
    assert ep.lib.ep_dispatch_bwd(C.byref(L), P, n, P, None, MIS, None, None) == \
        ep.EP_ERR_ALIGN
    assert ep.lib.ep_combine_bwd(C.byref(L), P, n, MIS, P2, None) == ep.EP_ERR_ALIGN
    assert ep.lib.ep_combine_bwd(C.byref(L), P, n, P, MIS, None) == ep.EP_ERR_ALIGN
    out = C.c_uint32(0)
    assert ep.lib.ep_read_status(MIS, C.byref(out), None) == ep.EP_ERR_ALIGN


def test_status_strings():
    for code in range(8):
        s = ep.status_str(code)
        assert s and s != "unknown ep_status_t"
    assert ep.status_str(99) == "unknown ep_status_t"


def test_binding_rejects_bad_tensors_on_cpu():
    import torch
    L = lay()
    h = torch.empty(ep.handle_mem_size(L), dtype=torch.uint8)
    with pytest.raises(TypeError):
        ep.prepare(L, torch.zeros((16, 2), dtype=torch.int32), torch.zeros(4, dtype=torch.int32), h)
    with pytest.raises(ValueError):   # not a GPU tensor
        ep.prepare(L, torch.zeros((16, 2), dtype=torch.int64), torch.zeros(4, dtype=torch.int32), h)


def test_weighted_entry_points_error_paths():
    # ep_combine_weighted(layout, handle, bytes, expert_out, recv_w, result, stream)
    # ep_combine_weighted_bwd(layout, handle, bytes, grad, expert_out, recv_w,
    #                         grad_expert_out, grad_recv_w, stream)
    cw, cwb = ep.lib.ep_combine_weighted, ep.lib.ep_combine_weighted_bwd
    L = lay()
    n = ep.handle_mem_size(L)
    bad = lay(K=0)
    assert cw(C.byref(bad), P, 1 << 30, P, P2, P2, None) == ep.EP_ERR_SHAPE
    assert cwb(C.byref(bad), P, 1 << 30, P, P2, P2, P2, P2, None) == ep.EP_ERR_SHAPE
    assert cw(None, P, n, P, P2, P2, None) == ep.EP_ERR_NULL
    assert cw(C.byref(L), None, n, P, P2, P2, None) == ep.EP_ERR_NULL
    assert cw(C.byref(L), P, n, None, P2, P2, None) == ep.EP_ERR_NULL      # rows
    assert cw(C.byref(L), P, n, P, None, P2, None) == ep.EP_ERR_NULL      # weights
    assert cw(C.byref(L), P, n, P, P2, None, None) == ep.EP_ERR_NULL      # result
    m = ep.handle_regions(L).maps_bytes       # the payload ops read the maps only
    assert cw(C.byref(L), P, m - 1, P, P2, P2, None) == ep.EP_ERR_HANDLE_SIZE
    assert cw(C.byref(L), P, n, MIS, P2, P2, None) == ep.EP_ERR_ALIGN
    assert cw(C.byref(L), P, n, P, P2, MIS, None) == ep.EP_ERR_ALIGN
    assert cwb(C.byref(L), P, n, None, P2, P2, P2, P2, None) == ep.EP_ERR_NULL   # grad
    assert cwb(C.byref(L), P, n, P, P2, None, P2, P2, None) == ep.EP_ERR_NULL   # weights
    assert cwb(C.byref(L), P, n, P, P2, P2, None, P2, None) == ep.EP_ERR_NULL   # grad rows
    # a weight gradient needs the expert rows
    assert cwb(C.byref(L), P, n, P, None, P2, P2, P2, None) == ep.EP_ERR_NULL
    assert cwb(C.byref(L), P, m - 1, P, P2, P2, P2, P2, None) == ep.EP_ERR_HANDLE_SIZE
    assert cwb(C.byref(L), P, n, MIS, P2, P2, P2, P2, None) == ep.EP_ERR_ALIGN
    assert cwb(C.byref(L), P, n, P, MIS, P2, P2, P2, None) == ep.EP_ERR_ALIGN
    assert cwb(C.byref(L), P, n, P, P2, P2, MIS, P2, None) == ep.EP_ERR_ALIGN


@pytest.mark.parametrize("flags", [0, 1, 4])
def test_token_buffers_required_even_without_receive_rows(flags):
    """A [T,...] buffer may be NULL only when T == 0: with tokens but no
    receive capacity the token-side pointers are still required, and the
    call fails before any HIP call (no kernel could read through them)."""
    L = lay(T=16, cap=0)
    L.flags = flags
    n = ep.handle_mem_size(L)
    assert n > 0
    # dispatch: tokens NULL, receive buffers NULL (allowed: cap == 0)
    assert ep.lib.ep_dispatch(C.byref(L), P, n, None, None, None, None, None) == \
        ep.EP_ERR_NULL
    # combine_bwd: gradient of the result NULL
    assert ep.lib.ep_combine_bwd(C.byref(L), P, n, None, None, None) == ep.EP_ERR_NULL
    # combine / dispatch_bwd: the [T,H] output NULL
    assert ep.lib.ep_combine(C.byref(L), P, n, None, None, None) == ep.EP_ERR_NULL
    assert ep.lib.ep_dispatch_bwd(C.byref(L), P, n, None, None, None, None, None) == \
        ep.EP_ERR_NULL
    # weighted backward: the [T,H] gradient NULL
    assert ep.lib.ep_combine_weighted_bwd(C.byref(L), P, n, None, None, None, None, None,
                                          None) == ep.EP_ERR_NULL


def test_receive_buffers_required_without_tokens():
    """With recv_capacity > 0 the [recv_capacity,...] inputs are required even
    when T == 0."""
    L = lay(T=0, cap=64)
    n = ep.handle_mem_size(L)
    assert ep.lib.ep_combine(C.byref(L), P, n, None, None, None) == ep.EP_ERR_NULL
    assert ep.lib.ep_dispatch_bwd(C.byref(L), P, n, None, None, None, None, None) == \
        ep.EP_ERR_NULL
    assert ep.lib.ep_combine_weighted(C.byref(L), P, n, None, None, None, None) == \
        ep.EP_ERR_NULL


def test_prepare_static_host_checks():
    """ep_prepare_static: the same argument checks as ep_prepare, a handle of
    the routing maps alone is enough, and a layout whose scratch exceeds the
    static array is refused with EP_ERR_SCRATCH, all before any HIP call."""
    fn = ep.lib.ep_prepare_static
    L = lay(T=4096, K=8, E=256, A=128, H=7168)
    m = ep.handle_regions(L).maps_bytes
    assert fn(C.byref(lay(K=0)), P, P, None, P, 1 << 30, None) == ep.EP_ERR_SHAPE
    assert fn(None, P, P, None, P, m, None) == ep.EP_ERR_NULL
    assert fn(C.byref(L), None, P, None, P, m, None) == ep.EP_ERR_NULL
    assert fn(C.byref(L), P, None, None, P, m, None) == ep.EP_ERR_NULL
    assert fn(C.byref(L), P, P, None, None, m, None) == ep.EP_ERR_NULL
    assert fn(C.byref(L), P, P, None, P, m - 1, None) == ep.EP_ERR_HANDLE_SIZE
    assert fn(C.byref(L), P, P, None, MIS, m, None) == ep.EP_ERR_ALIGN
    # 2^20 tokens x 8 routes over 2048 experts: 16384 units of 2048-entry
    # histograms, 128 MiB of scratch
    big = lay(T=1 << 20, K=8, E=2048, A=1, H=64, cap=64)
    assert ep.handle_mem_size(big) > 0
    assert fn(C.byref(big), P, P, None, P, 1 << 40, None) == ep.EP_ERR_SCRATCH
    assert "static" in ep.status_str(ep.EP_ERR_SCRATCH)
    # the largest layout it takes at E = 256: 4 MiB holds the 256-entry
    # histograms of 3614 units, of their 452 blocks of 8 and one totals row
    # (4067 KiB), plus two words per unit (28.25 KiB); 3615 units need 1 KiB
    # more rows, and with their words that is past 4 MiB
    for units, want_ok in ((3614, True), (3615, False)):
        Lu = lay(T=units * 64, K=8, E=256, A=1, H=64, cap=64)
        code = fn(C.byref(Lu), P, P, None, MIS, 1 << 40, None)
        assert code == (ep.EP_ERR_ALIGN if want_ok else ep.EP_ERR_SCRATCH)
