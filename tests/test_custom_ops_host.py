"""Host-side checks of the torch.library registration: every op is registered
under its schema, and the fake implementations give the right output shapes
and types without running anything (FakeTensorMode, no GPU)."""
import torch
from torch._subclasses.fake_tensor import FakeTensorMode

import combine_ep_prepare_amd as ep
from combine_ep_prepare_amd import custom_ops as cops

OPS = ["prepare", "dispatch", "dispatch_bwd", "combine", "combine_bwd", "combine_weighted",
       "combine_weighted_bwd"]


def test_ops_registered():
    for name in OPS:
        op = getattr(torch.ops.ep_mi355x, name)
        assert op.default._schema.name == f"ep_mi355x::{name}"
    sch = str(torch.ops.ep_mi355x.prepare.default._schema)
    assert "!) handle" in sch                  # prepare declares the handle mutated
    assert "!)" not in str(torch.ops.ep_mi355x.dispatch.default._schema)


def test_fake_shapes():
    T, K, E, A, H = 64, 4, 8, 16, 128
    cap = ep.recv_capacity_worst(T, K, E, A)
    for dt in ("bf16", "fp16", "fp32"):
        L = ep.Layout(T, K, E, A, H, cap, dtype=dt)
        ll = cops.layout_list(L)
        tdt = L.payload_dtype
        with FakeTensorMode():
            idx = torch.empty(T, K, dtype=torch.int64)
            handle = torch.empty(ep.handle_mem_size(L), dtype=torch.uint8)
            x = torch.empty(T, H, dtype=tdt)
            w = torch.empty(T, K)
            c, o = torch.ops.ep_mi355x.prepare(idx, handle, ll)
            assert c.shape == (E,) and o.shape == (E + 1,) and c.dtype == torch.int32
            recv, recv_w = torch.ops.ep_mi355x.dispatch(x, w, handle, ll)
            assert recv.shape == (cap, H) and recv.dtype == tdt and recv_w.shape == (cap,)
            gt, gw = torch.ops.ep_mi355x.dispatch_bwd(recv, None, handle, ll)
            assert gt.shape == (T, H) and gt.dtype == tdt and gw.shape == (T, K)
            y = torch.ops.ep_mi355x.combine(recv, handle, ll)
            assert y.shape == (T, H) and y.dtype == tdt
            g = torch.ops.ep_mi355x.combine_bwd(y, handle, ll)
            assert g.shape == (cap, H)
            yw = torch.ops.ep_mi355x.combine_weighted(recv, recv_w, handle, ll)
            assert yw.shape == (T, H)
            gr, gww = torch.ops.ep_mi355x.combine_weighted_bwd(yw, recv, recv_w, handle, ll)
            assert gr.shape == (cap, H) and gww.shape == (cap,) and gww.dtype == torch.float32


def test_layout_list_round_trip():
    L = ep.Layout(5, 2, 3, 4, 64, 100, dtype="fp32", fill_pads=False)
    ll = cops.layout_list(L)
    assert ll == [5, 2, 3, 4, 64, 100, ep.DTYPE_FP32, ep.LAYOUT_NO_PAD_FILL]
    L2 = cops._layout(ll)
    assert cops.layout_list(L2) == ll


def test_layout_flags_round_trip():
    # the pad and tail policies survive the op schema; the ops that allocate
    # an expert-major output add the tail policy
    for fill, tail in ((True, False), (False, False), (True, True), (False, True)):
        L = ep.Layout(16, 2, 4, 8, 64, 100, dtype="fp16", fill_pads=fill, zero_tail=tail)
        back = cops._layout(cops.layout_list(L))
        assert back.flags == L.flags and back.dtype == L.dtype
        assert cops.layout_list(back) == cops.layout_list(L)
        forced = cops._layout(cops.layout_list(L), zero_tail=True)
        assert forced.flags == L.flags | ep.LAYOUT_ZERO_TAIL
