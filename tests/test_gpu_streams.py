"""Handles in flight on several streams, and the allocation-free prepare in a
captured graph.

The per-step calls take the caller's stream and keep nothing between calls,
so several handles may be in flight at once ("Expert Parallelism: common C
API + NCCL EP backend", section "Per-step (allocation-free, CUDA-graph
capturable)"; the pipeline interleave of "[PyTorch] Expert Parallelism:
PyTorch wrapper + autograd ops with symm-mem zero-copy", section "Testing").
Two routings run their whole path on two streams at once, their launches
interleaved, and each must equal the oracle bit for bit. Then
ep_prepare_static, whose scratch is the library's static array, is captured
in a HIP graph with the payload ops on a handle of the routing maps alone and
replayed on new routings; every replay must equal an eager ep_prepare path.
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


class _Path:
    """One routing's buffers and its five ops on one stream."""

    def __init__(self, cfg, T, H, seed, stream):
        self.c = workloads.scaled(cfg, T=T, H=H)
        self.r = workloads.make_routing(self.c, seed)
        c = self.c
        self.cap = ep.recv_capacity_worst(T, c.K, c.E, c.A)
        self.L = ep.Layout(T, c.K, c.E, c.A, H, self.cap)
        self.stream = stream
        dev = "cuda"
        self.handle = ep.new_handle(self.L)
        self.idx = torch.from_numpy(self.r.topk_idx).to(dev)
        self.w = torch.from_numpy(self.r.topk_weights).to(dev)
        self.x = workloads.randn_bf16_torch((T, H), 10 + seed)
        self.y = workloads.randn_bf16_torch((self.cap, H), 20 + seed)
        self.g = workloads.randn_bf16_torch((T, H), 30 + seed)
        self.counts = torch.empty(c.E, dtype=torch.int32, device=dev)
        self.recv = torch.empty(self.cap, H, dtype=torch.bfloat16, device=dev)
        self.recv_w = torch.empty(self.cap, dtype=torch.float32, device=dev)
        self.res = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
        self.gx = torch.empty(self.cap, H, dtype=torch.bfloat16, device=dev)
        self.gt = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
        self.gw = torch.empty(T, c.K, dtype=torch.float32, device=dev)
        torch.cuda.synchronize()

    def ops(self):
        L, h, s = self.L, self.handle, self.stream
        return [lambda: ep.prepare(L, self.idx, self.counts, h, stream=s),
                lambda: ep.dispatch(L, h, self.x, self.w, self.recv, self.recv_w, stream=s),
                lambda: ep.combine(L, h, self.y, self.res, stream=s),
                lambda: ep.combine_bwd(L, h, self.g, self.gx, stream=s),
                lambda: ep.dispatch_bwd(L, h, self.y, self.recv_w, self.gt, self.gw, stream=s)]

    def check(self, label):
        p = oracle.prepare(self.r.topk_idx, self.c.E, self.c.A, self.cap)
        live = p.live
        assert np.array_equal(self.counts.cpu().numpy(), p.counts), label
        o_recv, o_w = oracle.dispatch(p, host_bf16(self.x), self.r.topk_weights)
        assert np.array_equal(host_bf16(self.recv)[:live], o_recv[:live]), label
        assert np.array_equal(self.recv_w.cpu().numpy()[:live].view(np.uint32),
                              o_w[:live].view(np.uint32)), label
        h_y = host_bf16(self.y)
        assert np.array_equal(host_bf16(self.res), oracle.combine(p, h_y)), label
        assert np.array_equal(host_bf16(self.gx)[:live],
                              oracle.combine_bwd(p, host_bf16(self.g))[:live]), label
        o_gt, o_gw = oracle.dispatch_bwd(p, h_y, self.recv_w.cpu().numpy())
        assert np.array_equal(host_bf16(self.gt), o_gt), label
        assert np.array_equal(self.gw.cpu().numpy().view(np.uint32), o_gw.view(np.uint32)), label
        assert ep.read_status(self.handle, stream=self.stream) == p.status, label


def test_two_streams_in_flight():
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()       # default priority
    a = _Path(workloads.CONFIGS["dsv3"], 2048, 1024, 1, s1)
    b = _Path(workloads.CONFIGS["qwen3"], 3000, 512, 2, s2)
    for rep in range(3):
        log(f"streams: round {rep}, two routings interleaved")
        for fa, fb in zip(a.ops(), b.ops()):
            fa()
            fb()
        torch.cuda.synchronize()
        a.check("dsv3 on stream 1")
        b.check("qwen3 on stream 2")


def test_prepare_static_in_a_graph():
    cfg = workloads.CONFIGS["dsv3"]
    T, H = 3000, 512
    cap = ep.recv_capacity_worst(T, cfg.K, cfg.E, cfg.A)
    L = ep.Layout(T, cfg.K, cfg.E, cfg.A, H, cap)
    regions = ep.handle_regions(L)
    dev = "cuda"

    def bufs(maps_only):
        n = regions.maps_bytes if maps_only else regions.bytes
        return dict(handle=torch.zeros(n, dtype=torch.uint8, device=dev),
                    idx=torch.zeros(T, cfg.K, dtype=torch.int64, device=dev),
                    w=torch.zeros(T, cfg.K, dtype=torch.float32, device=dev),
                    x=torch.zeros(T, H, dtype=torch.bfloat16, device=dev),
                    counts=torch.zeros(cfg.E, dtype=torch.int32, device=dev),
                    offsets=torch.zeros(cfg.E + 1, dtype=torch.int32, device=dev),
                    recv=torch.zeros(cap, H, dtype=torch.bfloat16, device=dev),
                    recv_w=torch.zeros(cap, dtype=torch.float32, device=dev),
                    res=torch.zeros(T, H, dtype=torch.bfloat16, device=dev))

    def run(b, static):
        prep = ep.prepare_static if static else ep.prepare
        prep(L, b["idx"], b["counts"], b["handle"], b["offsets"])
        ep.dispatch(L, b["handle"], b["x"], b["w"], b["recv"], b["recv_w"])
        ep.combine(L, b["handle"], b["recv"], b["res"])

    def fill(b, seed):
        r = workloads.make_routing(workloads.scaled(cfg, T=T, H=H), seed)
        b["idx"].copy_(torch.from_numpy(r.topk_idx))
        b["w"].copy_(torch.from_numpy(r.topk_weights))
        b["x"].copy_(workloads.randn_bf16_torch((T, H), 50 + seed))

    gb, eb = bufs(True), bufs(False)
    fill(gb, 0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(gb, True)                     # warm-up, outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(gb, True)
    torch.cuda.synchronize()
    for seed in range(1, 4):
        log(f"static prepare graph: replay with routing seed {seed}")
        fill(gb, seed)
        for k in ("idx", "w", "x"):
            eb[k].copy_(gb[k])
        run(eb, False)                    # eager, ep_prepare on a whole handle
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        live = min(int(eb["offsets"][-1].item()), cap)
        for k in ("counts", "offsets", "res"):
            assert torch.equal(gb[k].view(torch.uint8), eb[k].view(torch.uint8)), (seed, k)
        for k in ("recv", "recv_w"):
            assert torch.equal(gb[k][:live].view(torch.uint8), eb[k][:live].view(torch.uint8)), \
                (seed, k)
        assert ep.read_status(gb["handle"]) == ep.read_status(eb["handle"]) == 0
