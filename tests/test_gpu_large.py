"""GPU parity on receive buffers whose live rows lie past 2^31 and 2^32 bytes.

Every route local: T = 40960 tokens, each with 8 distinct experts of 32
drawn uniformly, H = 7168 bf16 (14 KiB rows), alignment 128. That gives
327 680 routes and about 331 000 live received rows, 4.7 GB: rows past
149 796 start beyond 2^31 bytes and rows past 299 593 beyond 2^32, so every
64-bit row offset in the run copy and the reduce is exercised. The
shape is the masked workload's (DeepSeek-V3 rows, a local slice of 32
experts) with no route masked, the largest receive buffer that slice can
need.

Each op is compared with the oracle element by element on the live rows, and
the rows past the live total are checked to still hold their canary.
"""
import dataclasses

import numpy as np
import pytest
import torch

import combine_ep_prepare_amd as ep
import oracle
import workloads
from gpu_harness import CANARY_BF16, CANARY_F32, bits32, host_bf16, log

pytestmark = pytest.mark.gpu

T_LARGE = 40960


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build()


@pytest.fixture(scope="module")
def case():
    cfg = dataclasses.replace(workloads.CONFIGS["masked"], name="all_local", T=T_LARGE,
                              routing="uniform", local_slice=None, global_E=None)
    r = workloads.make_routing(cfg)
    assert (r.topk_idx >= 0).all()
    cap = oracle.recv_capacity_worst(cfg.T, cfg.K, cfg.E, cfg.A)
    p = oracle.prepare(r.topk_idx, cfg.E, cfg.A, cap)
    B = cfg.H * 2
    assert p.live * B > 2 ** 32 and p.status == 0
    log(f"large: T={cfg.T} H={cfg.H} E={cfg.E} K={cfg.K} cap={cap} live={p.live} "
        f"({p.live * B / 1e9:.2f} GB)")
    return cfg, r, cap, p


def _canary_rows(n, H):
    t = torch.empty((n, H), dtype=torch.int16, device="cuda")
    t.fill_(np.array([CANARY_BF16], np.uint16).view(np.int16)[0].item())
    return t.view(torch.bfloat16)


def _tail_untouched(t, live):
    return bool((t[live:].view(torch.int16) ==
                 np.array([CANARY_BF16], np.uint16).view(np.int16)[0].item()).all())


def _prepared(cfg, r, cap, prepare_dtype):
    # prepare's chunk size follows its layout's row: bf16 rows give chunks
    # of 4 units, fp32 rows of 2; the payload ops use the bf16 layout
    L = ep.Layout(cfg.T, cfg.K, cfg.E, cfg.A, cfg.H, cap)
    Lp = ep.Layout(cfg.T, cfg.K, cfg.E, cfg.A, cfg.H, cap, dtype=prepare_dtype)
    handle = ep.new_handle(L)
    counts = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
    ep.prepare(Lp, torch.from_numpy(r.topk_idx).cuda(), counts, handle)
    return L, handle, counts


@pytest.mark.parametrize("prepare_dtype", ["bf16", "fp32"])
def test_large_dispatch_and_combine_bwd(case, prepare_dtype):
    cfg, r, cap, p = case
    L, handle, counts = _prepared(cfg, r, cap, prepare_dtype)
    m = ep.handle_maps(L, handle)
    assert np.array_equal(counts.cpu().numpy(), p.counts)
    assert np.array_equal(m["slot"].cpu().numpy(), p.slot)
    assert np.array_equal(m["row_src"][:p.live].cpu().numpy(), p.row_src[:p.live])
    live = p.live
    x = workloads.randn_bf16_torch((cfg.T, cfg.H), 31)
    w = torch.from_numpy(r.topk_weights).cuda()
    log(f"large prepared for {prepare_dtype}: dispatch")
    recv = _canary_rows(cap, cfg.H)
    recv_w = torch.full((cap,), float(CANARY_F32), device="cuda")
    ep.dispatch(L, handle, x, w, recv, recv_w)
    torch.cuda.synchronize()
    assert _tail_untouched(recv, live)
    assert (recv_w[live:] == float(CANARY_F32)).all()
    got = host_bf16(recv[:live])
    del recv
    want, want_w = oracle.dispatch(p, host_bf16(x), r.topk_weights)
    assert np.array_equal(got, want[:live]), "dispatch rows"
    assert np.array_equal(bits32(recv_w[:live].cpu().numpy()), bits32(want_w[:live]))
    del got, want
    log(f"large prepared for {prepare_dtype}: combine_bwd")
    g = workloads.randn_bf16_torch((cfg.T, cfg.H), 32)
    gx = _canary_rows(cap, cfg.H)
    ep.combine_bwd(L, handle, g, gx)
    torch.cuda.synchronize()
    assert _tail_untouched(gx, live)
    got = host_bf16(gx[:live])
    del gx
    want = oracle.combine_bwd(p, host_bf16(g))
    assert np.array_equal(got, want[:live]), "combine_bwd rows"
    assert ep.read_status(handle) == 0


def test_large_combine_and_dispatch_bwd(case):
    cfg, r, cap, p = case
    L, handle, _ = _prepared(cfg, r, cap, "bf16")
    live = p.live
    log("large: combine")
    Y = workloads.randn_bf16_torch((cap, cfg.H), 33)
    out = _canary_rows(cfg.T, cfg.H)
    ep.combine(L, handle, Y, out)
    torch.cuda.synchronize()
    Yh = host_bf16(Y[:live])          # combine reads live rows only
    del Y
    assert np.array_equal(host_bf16(out), oracle.combine(p, Yh)), "combine"
    del Yh, out
    log("large: dispatch_bwd")
    G = workloads.randn_bf16_torch((cap, cfg.H), 34)
    Gw = workloads.randn_bf16_torch((cap,), 35).float()
    gt = _canary_rows(cfg.T, cfg.H)
    gw = torch.full((cfg.T, cfg.K), float(CANARY_F32), device="cuda")
    ep.dispatch_bwd(L, handle, G, Gw, gt, gw)
    torch.cuda.synchronize()
    Gh = host_bf16(G[:live])
    del G
    o_gt, o_gw = oracle.dispatch_bwd(p, Gh, Gw[:live].cpu().numpy())
    assert np.array_equal(host_bf16(gt), o_gt), "dispatch_bwd tokens"
    assert np.array_equal(bits32(gw.cpu().numpy()), bits32(o_gw)), "dispatch_bwd weights"
    assert ep.read_status(handle) == 0
