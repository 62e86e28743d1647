"""Autograd dispatch/combine: forward + backward round trips and the VJP.

Follows the test list of "[PyTorch] Expert Parallelism: PyTorch wrapper +
autograd ops with symm-mem zero-copy", section "Testing": identity round trip,
dispatch forward+backward VJP, full forward+backward round trip, multi-
iteration bit stability, several routings in flight at once (a pipeline's
microbatches); and the None weight-gradient case of its review.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from combine_ep_prepare_amd import autograd as epa
from combine_ep_prepare_amd import handle_maps
from gpu_harness import host_bf16, wbwd_gamma

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build()


def _setup(name="dsv3", T=600, H=512, seed=0, small_ints=False):
    cfg = workloads.scaled(workloads.CONFIGS[name], T=T, H=H)
    r = workloads.make_routing(cfg, seed)
    if small_ints:
        rng = np.random.default_rng(seed)
        x = torch.from_numpy(workloads.small_int_bf16(rng, (T, H)).view(np.int16)).view(
            torch.bfloat16).cuda()
    else:
        x = workloads.randn_bf16_torch((T, H), 10 + seed)
    idx = torch.from_numpy(r.topk_idx).cuda()
    w = torch.from_numpy(r.topk_weights).cuda()
    return cfg, r, idx, x, w


def test_identity_round_trip_and_none_weight_grad():
    cfg, r, idx, x, w = _setup(small_ints=True)
    routing = epa.EpRouting(idx, cfg.E, cfg.A, cfg.H)
    x = x.clone().requires_grad_(True)
    w = w.clone().requires_grad_(True)
    recv, recv_w = epa.dispatch(x, w, routing)
    y = epa.combine(recv, routing)              # identity experts, weights unused
    n = (r.topk_idx >= 0).sum(axis=1)
    want = (x.detach().float() * torch.from_numpy(n).cuda()[:, None].float()).to(torch.bfloat16)
    assert torch.equal(y.view(torch.int16), want.view(torch.int16))
    g = torch.from_numpy(workloads.small_int_bf16(np.random.default_rng(5),
                                                  (cfg.T, cfg.H)).view(np.int16)).view(
        torch.bfloat16).cuda()
    y.backward(g)
    # d(combine(dispatch(x)))/dx applied to g is n_valid * g, exactly for small ints
    want_g = (g.float() * torch.from_numpy(n).cuda()[:, None].float()).to(torch.bfloat16)
    assert torch.equal(x.grad.view(torch.int16), want_g.view(torch.int16))
    # no gradient reached the received weights: the weight gradient is zero
    assert w.grad is not None and torch.count_nonzero(w.grad) == 0


@pytest.mark.parametrize("zero_tail", [False, True])
def test_weighted_round_trip_grads_match_oracle(zero_tail):
    cfg, r, idx, x, w = _setup(name="qwen3", T=500, H=256, seed=1)
    routing = epa.EpRouting(idx, cfg.E, cfg.A, cfg.H, zero_tail=zero_tail)
    x = x.clone().requires_grad_(True)
    w = w.clone().requires_grad_(True)
    recv, recv_w = epa.dispatch(x, w, routing)
    recv.retain_grad()
    recv_w.retain_grad()
    expert_out = (recv.float() * recv_w[:, None]).to(torch.bfloat16)   # caller's pre-multiply
    y = epa.combine(expert_out, routing)
    g = workloads.randn_bf16_torch((cfg.T, cfg.H), 77)
    (y.float() * g.float()).sum().backward()
    p = oracle.prepare(r.topk_idx, cfg.E, cfg.A, routing.layout.cap)
    live = p.live
    # forward
    o_recv, o_recv_w = oracle.dispatch(p, host_bf16(x.detach()), r.topk_weights)
    assert np.array_equal(host_bf16(recv.detach())[:live], o_recv[:live])
    assert np.array_equal(recv_w.detach().cpu().numpy()[:live].view(np.uint32),
                          o_recv_w[:live].view(np.uint32))
    assert np.array_equal(host_bf16(y.detach()), oracle.combine(p, host_bf16(expert_out)))
    # backward: the token and weight grads are dispatch_bwd of what reached recv
    g_recv = host_bf16(recv.grad)
    g_recv_w = recv_w.grad.cpu().numpy()
    o_gt, o_gw = oracle.dispatch_bwd(p, g_recv, g_recv_w)
    assert np.array_equal(host_bf16(x.grad), o_gt)
    assert np.array_equal(w.grad.cpu().numpy().view(np.uint32), o_gw.view(np.uint32))
    # and recv.grad itself came from combine_bwd of g, then the multiply's backward
    m = handle_maps(routing.layout, routing.handle)
    slot = m["slot"].cpu().numpy()
    assert (slot[(r.topk_idx < 0).reshape(-1)] == -1).all()


def test_bit_stable_and_interleaved_routings():
    # three routings in flight at once (as a pipeline's microbatches would be),
    # run in interleaved order, repeated: results are bit-identical each time
    states = [_setup(name="dsv3", T=300 + 50 * i, H=256, seed=i) for i in range(3)]
    first = None
    for rep in range(3):
        routings = [epa.EpRouting(idx, cfg.E, cfg.A, cfg.H) for cfg, r, idx, x, w in states]
        recvs = [epa.dispatch(s[3], s[4], rt)[0] for s, rt in zip(states, routings)]
        outs = [epa.combine(rv, rt) for rv, rt in zip(reversed(recvs), reversed(routings))]
        outs = [o.clone() for o in reversed(outs)]
        if first is None:
            first = outs
        else:
            for a, b in zip(first, outs):
                assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    for (cfg, r, idx, x, w), o in zip(states, first):
        n = torch.from_numpy((r.topk_idx >= 0).sum(axis=1)).cuda()
        want = (x.float() * n[:, None].float()).to(torch.bfloat16)
        assert torch.equal(o.view(torch.int16), want.view(torch.int16))


def test_fused_weighted_combine_grads():
    # combine with the weights applied inside: forward bit-exact, the row grads
    # and token grads bit-exact, the weight grads within the dot's fp32 bound
    cfg, r, idx, x, w = _setup(name="dsv3", T=400, H=1024, seed=2)
    routing = epa.EpRouting(idx, cfg.E, cfg.A, cfg.H)
    x = x.clone().requires_grad_(True)
    w = w.clone().requires_grad_(True)
    recv, recv_w = epa.dispatch(x, w, routing)
    recv.retain_grad()
    recv_w.retain_grad()
    y = epa.combine(recv, routing, recv_w)          # identity experts, fused weights
    g = workloads.randn_bf16_torch((cfg.T, cfg.H), 78)
    y.backward(g)
    p = oracle.prepare(r.topk_idx, cfg.E, cfg.A, routing.layout.cap)
    live = p.live
    h_recv = host_bf16(recv.detach())
    h_recv_w = recv_w.detach().cpu().numpy()
    assert np.array_equal(host_bf16(y.detach()), oracle.combine_weighted(p, h_recv, h_recv_w))
    o_gr, o_gw, o_abs = oracle.combine_weighted_bwd(p, host_bf16(g), h_recv, h_recv_w)
    assert np.array_equal(host_bf16(recv.grad)[:live], o_gr[:live])
    got = recv_w.grad.cpu().numpy()[:live].astype(np.float64)
    assert (np.abs(got - o_gw[:live]) <= wbwd_gamma(cfg.H) * o_abs[:live] + 1e-45).all()
    # then through dispatch's backward, bit for bit
    o_gt, o_gwt = oracle.dispatch_bwd(p, host_bf16(recv.grad), recv_w.grad.cpu().numpy())
    assert np.array_equal(host_bf16(x.grad), o_gt)
    assert np.array_equal(w.grad.cpu().numpy().view(np.uint32), o_gwt.view(np.uint32))


@pytest.mark.parametrize("dt", ["fp16", "fp32"])
def test_payload_types_through_autograd(dt):
    # the same routing serves every payload type; forward and token/weight
    # gradients against the oracle's fp16 / fp32 paths
    cfg, r, idx, x, w = _setup(name="qwen3", T=300, H=256, seed=4)
    tdt = {"fp16": torch.float16, "fp32": torch.float32}[dt]
    routing = epa.EpRouting(idx, cfg.E, cfg.A, cfg.H, fill_pads=False)
    xt = x.float().to(tdt).clone().requires_grad_(True)
    wt = w.clone().requires_grad_(True)
    recv, recv_w = epa.dispatch(xt, wt, routing)
    recv.retain_grad()
    y = epa.combine(recv, routing, recv_w)
    g = workloads.randn_bf16_torch((cfg.T, cfg.H), 80).float().to(tdt)
    y.backward(g)
    p = oracle.prepare(r.topk_idx, cfg.E, cfg.A, routing.layout.cap)
    live = p.live

    def h(t):
        t = t.detach()
        return (t.cpu().numpy() if dt == "fp32"
                else t.view(torch.int16).cpu().numpy().view(np.uint16))

    def bits(a):
        return a.view(np.uint32) if a.dtype == np.float32 else a

    o_recv, o_recv_w = oracle.dispatch(p, h(xt), r.topk_weights, dtype=dt, fill_pads=False)
    pad = p.row_src[:live] < 0
    assert np.array_equal(bits(h(recv)[:live][~pad]), bits(o_recv[:live][~pad]))
    # pad rows were never written: combine reads only the rows of valid routes
    rw = recv_w.detach().cpu().numpy()          # weights are fp32 for every payload type
    assert np.array_equal(bits(h(y)), bits(oracle.combine_weighted(p, h(recv), rw, dtype=dt)))
    o_gr, _, _ = oracle.combine_weighted_bwd(p, h(g), h(recv), rw, dtype=dt, fill_pads=False)
    assert np.array_equal(bits(h(recv.grad)[:live][~pad]), bits(o_gr[:live][~pad]))
    o_gt, _ = oracle.dispatch_bwd(p, h(recv.grad), None, want_grad_w=False, dtype=dt)
    assert np.array_equal(bits(h(xt.grad)), bits(o_gt))
    assert wt.grad is not None and wt.grad.shape == (cfg.T, cfg.K)


@pytest.mark.parametrize("weighted", [False, True])
def test_shared_expert_over_whole_buffer_gets_exact_grads(weighted):
    # One Linear-style expert applied to the whole [cap,H] receive buffer (a
    # parameter shared by every row). Its weight gradient sums over all rows,
    # so it is only right if every row the routing does not fill (pads and
    # the tail past the live total) carries zeros forward and a zero
    # gradient back. The buffers are allocated uninitialised and filled with
    # NaN beforehand, so stale memory would show. The reference takes the
    # live rows only.
    cfg, r, idx, x, w = _setup(name="masked", T=900, H=256, seed=3)
    torch.cuda.synchronize()
    junk = torch.full((1 << 24,), float("nan"), device="cuda")   # poison the allocator's
    del junk                                                      # free blocks with NaN
    routing = epa.EpRouting(idx, cfg.E, cfg.A, cfg.H)
    cap = routing.layout.cap
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4)
    W = (torch.randn(cfg.H, cfg.H, generator=gen, device="cuda") / 16).requires_grad_(True)
    recv, recv_w = epa.dispatch(x, w, routing)
    h = (recv.float() @ W).to(torch.bfloat16)                   # the shared expert
    y = epa.combine(h, routing, recv_w if weighted else None)
    g = workloads.randn_bf16_torch((cfg.T, cfg.H), 78)
    (y.float() * g.float()).sum().backward()
    assert torch.isfinite(W.grad).all()
    live = int(routing.expert_offsets[-1].item())
    assert live < cap                   # the worst-case buffer has a tail
    # reference: the same expert on the live rows only, in fp32 on the CPU
    recv_l = recv.detach()[:live].float().cpu()
    W_c = W.detach().cpu()
    h_l = (recv_l @ W_c).to(torch.bfloat16).requires_grad_(True)
    p = oracle.prepare(r.topk_idx, cfg.E, cfg.A, cap)
    # d(sum(y*g))/dh on the live rows: combine_bwd of g (weighted: times w)
    gh = torch.from_numpy(oracle.combine_bwd(p, host_bf16(g))[:live].view(np.int16)).view(
        torch.bfloat16).float()
    if weighted:
        gh = (gh * recv_w.detach()[:live].cpu()[:, None]).to(torch.bfloat16).float()
    want = recv_l.t() @ gh
    got = W.grad.cpu()
    # the same products; only the summation order of the two GEMMs differs
    assert torch.allclose(got, want, rtol=1e-3, atol=1e-3 * want.abs().max().item())
