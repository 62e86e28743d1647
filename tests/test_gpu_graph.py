"""The whole path captured in a HIP graph and replayed.

The per-step calls are allocation-free and never synchronise ("[PyTorch]
Expert Parallelism: PyTorch wrapper + autograd ops with symm-mem zero-copy",
section "Testing": CUDA graph capture; "Expert Parallelism: common C API +
NCCL EP backend", section "Per-step (allocation-free, CUDA-graph
capturable)"). The graph is replayed several times on new routing and new
token rows written into its static input buffers, with eager work and
synchronisations in between, and every replay is compared bit for bit with an
eager run and with the oracle.
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


class Step:
    """Static buffers of one step: prepare, dispatch, combine, combine_bwd,
    dispatch_bwd on a fixed layout."""

    def __init__(self, L: ep.Layout):
        d = "cuda"
        self.L = L
        self.handle = ep.new_handle(L)
        self.idx = torch.zeros(L.T, L.K, dtype=torch.int64, device=d)
        self.w = torch.zeros(L.T, L.K, dtype=torch.float32, device=d)
        self.x = torch.zeros(L.T, L.H, dtype=torch.bfloat16, device=d)
        self.expert_out = torch.zeros(L.cap, L.H, dtype=torch.bfloat16, device=d)
        self.g_res = torch.zeros(L.T, L.H, dtype=torch.bfloat16, device=d)
        self.g_recv = torch.zeros(L.cap, L.H, dtype=torch.bfloat16, device=d)
        self.g_recv_w = torch.zeros(L.cap, dtype=torch.float32, device=d)
        self.counts = torch.zeros(L.E, dtype=torch.int32, device=d)
        self.offsets = torch.zeros(L.E + 1, dtype=torch.int32, device=d)
        self.recv = torch.zeros(L.cap, L.H, dtype=torch.bfloat16, device=d)
        self.recv_w = torch.zeros(L.cap, dtype=torch.float32, device=d)
        self.res = torch.zeros(L.T, L.H, dtype=torch.bfloat16, device=d)
        self.g_exp = torch.zeros(L.cap, L.H, dtype=torch.bfloat16, device=d)
        self.g_tok = torch.zeros(L.T, L.H, dtype=torch.bfloat16, device=d)
        self.g_w = torch.zeros(L.T, L.K, dtype=torch.float32, device=d)

    def run(self):
        L = self.L
        ep.prepare(L, self.idx, self.counts, self.handle, self.offsets)
        ep.dispatch(L, self.handle, self.x, self.w, self.recv, self.recv_w)
        ep.combine(L, self.handle, self.expert_out, self.res)
        ep.combine_bwd(L, self.handle, self.g_res, self.g_exp)
        ep.dispatch_bwd(L, self.handle, self.g_recv, self.g_recv_w, self.g_tok, self.g_w)

    def load(self, other: "Step"):
        for name in ("idx", "w", "x", "expert_out", "g_res", "g_recv", "g_recv_w"):
            getattr(self, name).copy_(getattr(other, name))

    def outputs(self):
        return [self.counts, self.offsets, self.recv, self.recv_w, self.res, self.g_exp,
                self.g_tok, self.g_w]


def _fill(step: Step, cfg, seed: int):
    c = workloads.scaled(cfg, T=step.L.T, H=step.L.H)
    r = workloads.make_routing(c, seed)
    step.idx.copy_(torch.from_numpy(r.topk_idx))
    step.w.copy_(torch.from_numpy(r.topk_weights))
    step.x.copy_(workloads.randn_bf16_torch((step.L.T, step.L.H), 100 + seed))
    step.expert_out.copy_(workloads.randn_bf16_torch((step.L.cap, step.L.H), 200 + seed))
    step.g_res.copy_(workloads.randn_bf16_torch((step.L.T, step.L.H), 300 + seed))
    step.g_recv.copy_(workloads.randn_bf16_torch((step.L.cap, step.L.H), 400 + seed))
    step.g_recv_w.copy_(workloads.randn_bf16_torch((step.L.cap,), 500 + seed).float())
    return r


def _same(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


# dsv3 at T=700 and masked_hot take the two-kernel prepare; tiny and dsv3 at
# T=400 (at most 4096 routes) the one-block prepare; zero_tail: the rows past
# the live total are zeroed on every replay too
@pytest.mark.parametrize("name,T,H,zero_tail", [
    ("dsv3", 700, 1024, False), ("masked_hot", 2048, 512, False), ("tiny", 256, 512, False),
    ("dsv3", 400, 1024, False), ("dsv3", 700, 1024, True), ("tiny", 256, 512, True),
    ("masked_hot", 2048, 512, True)])
def test_graph_replays_match_eager_and_oracle(name, T, H, zero_tail):
    cfg = workloads.CONFIGS[name]
    cap = ep.recv_capacity_worst(T, cfg.K, cfg.E, cfg.A)
    L = ep.Layout(T, cfg.K, cfg.E, cfg.A, H, cap, zero_tail=zero_tail)
    g_step, e_step = Step(L), Step(L)
    _fill(g_step, cfg, 0)
    # warm up on a side stream, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g_step.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g_step.run()
    torch.cuda.synchronize()
    for seed in range(1, 5):
        log(f"graph {name}: replay with routing seed {seed}")
        r = _fill(g_step, cfg, seed)
        e_step.load(g_step)
        e_step.run()                      # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        # receive-side outputs are defined on live rows only (rows past the
        # live total keep what an earlier routing left there), on every row
        # under the tail policy, which zeroes the tail
        live = min(int(e_step.offsets[-1].item()), cap)
        for a, b in zip(g_step.outputs(), e_step.outputs()):
            if a.shape[0] == cap and cap != L.T:
                if zero_tail:
                    assert not a[live:].view(torch.uint8).any(), f"replay {seed}: tail"
                else:
                    a, b = a[:live], b[:live]
            assert _same(a, b), f"replay {seed} differs from eager"
        assert ep.read_status(g_step.handle) == 0
        if seed == 2:
            p = oracle.prepare(r.topk_idx, L.E, L.A, cap)
            assert np.array_equal(g_step.counts.cpu().numpy(), p.counts)
            live = p.live
            o_recv, _ = oracle.dispatch(p, host_bf16(g_step.x), r.topk_weights)
            assert np.array_equal(host_bf16(g_step.recv)[:live], o_recv[:live])
            assert np.array_equal(host_bf16(g_step.res),
                                  oracle.combine(p, host_bf16(g_step.expert_out)))


@pytest.mark.parametrize("dt,fill,alternate", [("fp32", False, False), ("fp16", True, False),
                                              ("bf16", True, True)])
def test_graph_weighted_ops_other_payload_types(dt, fill, alternate):
    # prepare, dispatch, weighted combine and its backward captured on an
    # fp32 layout without the pad fill (and fp16 with it); every replay on new
    # routing equals an eager run bit for bit, the weight gradient included.
    # With `alternate`, odd replays mask 85% of the routes, so the backward's
    # walk (received rows on sparse routings, run lists on dense ones),
    # chosen on the device, changes from replay to replay of one graph.
    cfg = workloads.CONFIGS["qwen3"]
    T, H = 600, 512
    cap = ep.recv_capacity_worst(T, cfg.K, cfg.E, cfg.A)
    L = ep.Layout(T, cfg.K, cfg.E, cfg.A, H, cap, dtype=dt, fill_pads=fill)
    tdt = L.payload_dtype

    def bufs():
        z = lambda *s, dtype=tdt: torch.zeros(*s, dtype=dtype, device="cuda")  # noqa: E731
        return dict(handle=ep.new_handle(L), idx=z(T, cfg.K, dtype=torch.int64),
                    w=z(T, cfg.K, dtype=torch.float32), x=z(T, H), g=z(T, H),
                    counts=z(cfg.E, dtype=torch.int32), recv=z(cap, H),
                    recv_w=z(cap, dtype=torch.float32), y=z(T, H), gr=z(cap, H),
                    gw=z(cap, dtype=torch.float32))

    def run(b):
        ep.prepare(L, b["idx"], b["counts"], b["handle"])
        ep.dispatch(L, b["handle"], b["x"], b["w"], b["recv"], b["recv_w"])
        ep.combine_weighted(L, b["handle"], b["recv"], b["recv_w"], b["y"])
        ep.combine_weighted_bwd(L, b["handle"], b["g"], b["recv"], b["recv_w"], b["gr"], b["gw"])

    def fill_inputs(b, seed):
        c = workloads.scaled(cfg, T=T, H=H)
        r = workloads.make_routing(c, seed)
        idx = r.topk_idx.copy()
        if alternate and seed % 2:
            idx[np.random.default_rng(seed).random(idx.shape) < 0.85] = -1
        b["idx"].copy_(torch.from_numpy(idx))
        b["w"].copy_(torch.from_numpy(r.topk_weights))
        b["x"].copy_(workloads.randn_bf16_torch((T, H), 600 + seed).to(tdt))
        b["g"].copy_(workloads.randn_bf16_torch((T, H), 700 + seed).to(tdt))

    gb, eb = bufs(), bufs()
    fill_inputs(gb, 0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(gb)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(gb)
    torch.cuda.synchronize()
    for seed in range(1, 4):
        log(f"graph weighted {dt}: replay with routing seed {seed}")
        fill_inputs(gb, seed)
        for k in ("idx", "w", "x", "g"):
            eb[k].copy_(gb[k])
        run(eb)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        # rows the ops define: live rows, pads only when they are filled (the
        # graph's buffers also hold rows of the warm-up routing elsewhere)
        maps = ep.handle_maps(L, eb["handle"])
        row_src = maps["row_src"]
        total = int(maps["offsets"][-1].item())
        live = min(total, cap)
        keep = row_src[:live] >= 0 if not fill else torch.ones(live, dtype=torch.bool,
                                                                 device="cuda")
        for k in ("counts", "y"):
            assert _same(gb[k], eb[k]), f"replay {seed}: {k} differs from eager"
        for k in ("recv", "recv_w", "gr", "gw"):
            assert _same(gb[k][:live][keep], eb[k][:live][keep]), \
                f"replay {seed}: {k} differs from eager"
