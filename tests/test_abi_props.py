"""Randomised host-side properties of the C ABI's size queries (no GPU).

For any valid layout the handle regions lie in the documented order, each
on a 256-byte boundary, the routing maps close at maps_bytes and prepare's
scratch fills the rest with exactly the sizes ep.h states; the handle does
not depend on the payload type, the flags or the row length, and grows with
the capacity. Any invalid layout is refused by the size queries and, before
any device pointer could be touched, by every call that takes it (the
pointers passed are fake and never dereferenced).
"""
import ctypes as C

import pytest
from hypothesis import given, settings, strategies as st

import combine_ep_prepare_amd as ep

P = C.c_void_p(0x10000)            # a fake, aligned device address


def a256(n):
    return (n + 255) // 256 * 256


@st.composite
def valid_layouts(draw):
    K = draw(st.integers(1, 64))
    E = draw(st.integers(1, 2048))
    A = draw(st.integers(1, 256))
    T = draw(st.integers(0, 300_000))
    if T * K + E * (A - 1) >= 1 << 31:
        T = ((1 << 31) - 1 - E * (A - 1)) // K
    H = 8 * draw(st.integers(1, 8192))
    worst = T * min(K, E) + E * (A - 1)
    cap = draw(st.integers(0, min(worst + 1000, (1 << 31) - 1)))
    dtype = draw(st.sampled_from(["bf16", "fp16", "fp32"]))
    fill = draw(st.booleans())
    tail = draw(st.booleans())
    return ep.Layout(T, K, E, A, H, cap, dtype=dtype, fill_pads=fill, zero_tail=tail)


@settings(max_examples=300, deadline=None)
@given(valid_layouts())
def test_regions_of_any_valid_layout(L):
    n = ep.handle_mem_size(L)
    assert n > 0
    r = ep.handle_regions(L)
    assert r.bytes == n
    T, K, E, cap = L.T, L.K, L.E, L.cap
    U = -(-(T * K) // 512)
    # the documented order, each region on a 256-byte boundary
    order = [r.counts, r.offsets, r.slot, r.row_src, r.runs, r.maps_bytes]
    assert all(x % 256 == 0 for x in order)
    assert r.status < 256 and r.stream_live < 256 and r.run_units < 256   # in the header
    assert order == sorted(order)
    assert r.offsets - r.counts >= 4 * E
    assert r.slot - r.offsets >= 4 * (E + 1)
    assert r.row_src - r.slot >= 4 * T * K
    assert r.runs - r.row_src >= 4 * cap
    # the run lists close the maps: 8 lists of 64 U + 2048 entries of 8 bytes
    assert r.run_list_entries == 64 * U + 2048
    assert r.maps_bytes - r.runs == a256(8 * 8 * r.run_list_entries)
    # prepare's scratch closes the handle: histogram rows (units, blocks of
    # 4 units up to 256 units and of 8 past that, a totals row) and two
    # words per unit
    blocks = -(-U // 4) if U <= 256 else -(-U // 8)
    assert n - r.maps_bytes == a256(4 * E * (U + blocks + 1)) + a256(8 * U)
    # nothing but T, K, E, A and the capacity sizes the handle
    for dt in ("bf16", "fp16", "fp32"):
        other = ep.Layout(T, K, E, L.A, 8, cap, dtype=dt)
        assert ep.handle_mem_size(other) == n
    if cap + 4096 < 1 << 31:
        bigger = ep.Layout(T, K, E, L.A, L.H, cap + 4096)
        assert ep.handle_mem_size(bigger) > n


@st.composite
def invalid_layouts(draw):
    T, K, E, A, H, cap = 100, 4, 16, 8, 64, 1000
    dtype, flags = 0, 0
    what = draw(st.sampled_from(["T", "K", "E", "A", "H", "cap", "dtype", "flags",
                                 "offsets"]))
    if what == "T":
        T = draw(st.integers(-(1 << 40), -1))
    elif what == "K":
        K = draw(st.one_of(st.integers(-100, 0), st.integers(65, 10_000)))
    elif what == "E":
        E = draw(st.one_of(st.integers(-100, 0), st.integers(2049, 1 << 20)))
    elif what == "A":
        A = draw(st.integers(-100, 0))
    elif what == "H":
        H = draw(st.one_of(st.integers(-64, 7), st.integers(9, 10_000).filter(lambda h: h % 8)))
    elif what == "cap":
        cap = draw(st.one_of(st.integers(-(1 << 40), -1), st.integers(1 << 31, 1 << 40)))
    elif what == "dtype":
        dtype = draw(st.integers(3, 0xFFFF))
    elif what == "flags":
        flags = draw(st.integers(1, 0xFFFF).filter(lambda f: f & ~0x5))
    else:   # T*K + E*(A-1) past int32 offsets
        T, K = (1 << 31) // 4, 4
    L = ep.Layout(T, K, E, A, H, cap, dtype=dtype)
    L.flags = flags
    return L


@settings(max_examples=300, deadline=None)
@given(invalid_layouts())
def test_invalid_layouts_are_refused_before_any_hip_call(L):
    assert ep.handle_mem_size(L) == 0
    out = ep.HandleRegions()
    assert ep.lib.ep_handle_regions(C.byref(L), C.byref(out)) != ep.EP_OK
    big = C.c_size_t(1 << 40)
    codes = [
        ep.lib.ep_prepare(C.byref(L), P, P, None, P, big, None),
        ep.lib.ep_prepare_static(C.byref(L), P, P, None, P, big, None),
        ep.lib.ep_dispatch(C.byref(L), P, big, P, None, P, None, None),
        ep.lib.ep_combine(C.byref(L), P, big, P, P, None),
        ep.lib.ep_combine_bwd(C.byref(L), P, big, P, P, None),
        ep.lib.ep_dispatch_bwd(C.byref(L), P, big, P, None, P, None, None),
        ep.lib.ep_combine_weighted(C.byref(L), P, big, P, P, P, None),
        ep.lib.ep_combine_weighted_bwd(C.byref(L), P, big, P, P, P, P, P, None),
    ]
    assert all(c not in (ep.EP_OK, ep.EP_ERR_HIP, ep.EP_ERR_DEVICE) for c in codes), codes
