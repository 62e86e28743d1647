"""ep_prepare_static against ep_prepare, through the C ABI.

The variant keeps prepare's scratch in the library's static device array, so
its handle holds the routing maps alone. Calls in a row, each with a smaller
routing than the last: one large enough for the column-scan prepare, two
for the two-kernel prepare (all three use the scratch), then a small one
that takes the one-block prepare: every
routing map and every payload op run from the variant's handle must equal,
bit for bit, what the same calls give from ep_prepare's handle, and the
oracle's maps.
"""
import numpy as np
import pytest
import torch

import combine_ep_prepare_amd as ep
import oracle
import workloads
from gpu_harness import host_bf16, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build()


def _maps(L, handle, live):
    m = ep.handle_maps(L, handle)
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in m.items()}
    out["row_src"] = out["row_src"][:live]
    # each run list up to its length (the rest of the region is not written)
    out["runs"] = np.concatenate([out["runs"][x, :out["stream_live"][x]] for x in range(8)])
    return out


# the payload type sizes the run chunks (fp32 rows: half the routes a chunk)
@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_prepare_static_matches_prepare(dt):
    # 40000 tokens of top-8: 625 units, past the 64 histogram-block rows, so
    # the column scan (and its chunk starts) runs in the static array too
    for name, T, H in (("dsv3", 40000, 256), ("dsv3", 4096, 1024), ("masked_hot", 1500, 512),
                       ("tiny", 256, 512)):
        cfg = workloads.scaled(workloads.CONFIGS[name], T=T, H=H)
        r = workloads.make_routing(cfg)
        cap = ep.recv_capacity_worst(T, cfg.K, cfg.E, cfg.A)
        L = ep.Layout(T, cfg.K, cfg.E, cfg.A, H, cap, dtype=dt)
        regions = ep.handle_regions(L)
        log(f"prepare_static {name}: T={T} K={cfg.K} E={cfg.E} routes={T * cfg.K} "
            f"maps {regions.maps_bytes} of {regions.bytes} bytes")
        idx = torch.from_numpy(r.topk_idx).cuda()
        # reference: ep_prepare into a whole handle
        h_ref = ep.new_handle(L)
        c_ref = torch.full((cfg.E,), -5, dtype=torch.int32, device="cuda")
        o_ref = torch.full((cfg.E + 1,), -5, dtype=torch.int32, device="cuda")
        ep.prepare(L, idx, c_ref, h_ref, o_ref)
        # the variant: a handle of the maps alone, filled with junk first
        h_st = torch.full((regions.maps_bytes,), 0xA5, dtype=torch.uint8, device="cuda")
        c_st = torch.full((cfg.E,), -6, dtype=torch.int32, device="cuda")
        o_st = torch.full((cfg.E + 1,), -6, dtype=torch.int32, device="cuda")
        ep.prepare_static(L, idx, c_st, h_st, o_st)
        p = oracle.prepare(r.topk_idx, cfg.E, cfg.A, cap)
        assert torch.equal(c_ref, c_st) and torch.equal(o_ref, o_st)
        assert np.array_equal(c_st.cpu().numpy(), p.counts)
        assert np.array_equal(o_st.cpu().numpy(), p.offsets)
        a, b = _maps(L, h_ref, p.live), _maps(L, h_st, p.live)
        for k in a:
            assert np.array_equal(a[k], b[k]), f"{name}: {k}"
        assert np.array_equal(b["slot"], p.slot)
        assert np.array_equal(b["row_src"], p.row_src[:p.live])
        assert ep.read_status(h_st) == p.status == ep.read_status(h_ref)
        # every payload op run from either handle gives the same bits (a
        # handle serves every payload type: bf16 payloads here)
        Lb = ep.Layout(T, cfg.K, cfg.E, cfg.A, H, cap)
        x = workloads.randn_bf16_torch((T, H), 40)
        w = torch.from_numpy(r.topk_weights).cuda()
        Y = workloads.randn_bf16_torch((cap, H), 41)
        outs = []
        for h in (h_ref, h_st):
            recv = torch.zeros(cap, H, dtype=torch.bfloat16, device="cuda")
            recv_w = torch.zeros(cap, device="cuda")
            ep.dispatch(Lb, h, x, w, recv, recv_w)
            res = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
            ep.combine(Lb, h, Y, res)
            gx = torch.zeros(cap, H, dtype=torch.bfloat16, device="cuda")
            ep.combine_bwd(Lb, h, x, gx)
            gt = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
            gw = torch.empty(T, cfg.K, device="cuda")
            ep.dispatch_bwd(Lb, h, Y, recv_w, gt, gw)
            outs.append([recv, recv_w, res, gx, gt, gw])
        torch.cuda.synchronize()
        for u, v in zip(*outs):
            assert torch.equal(u.view(torch.uint8), v.view(torch.uint8)), name
        want, _ = oracle.dispatch(p, host_bf16(x), r.topk_weights)
        assert np.array_equal(host_bf16(outs[1][0])[:p.live], want[:p.live])
