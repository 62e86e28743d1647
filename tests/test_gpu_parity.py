"""GPU parity: every op through the C ABI against the CPU oracle, bit for bit.

Sizes: every workload at a reduced token count that still spans many work
items and a ragged tail, the small workload and the four large ones at their
full sizes (the configuration the benchmark times), and the edge cases of the
method (no tokens, everything masked, one expert, no padding, generic top-k,
odd hidden sizes, many experts, repeated ids, bad ids, overflow).
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_harness import (CANARY_BF16, GpuRun, bits32, check_all_ops, check_prepare,
                         dev_bf16, dev_f32, host_bf16, host_f32, log)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build()


def _inputs(cfg, T, H, cap, seed=0, rows_kind="random"):
    c = workloads.scaled(cfg, T=T, H=H)
    r = workloads.make_routing(c, seed)
    x = workloads.make_tokens(c, seed)
    g_result, g_recv, g_recv_w = workloads.make_grads(c, cap, seed)
    rows = workloads.make_expert_rows(c, cap, seed)
    return c, r, x, rows, g_result, g_recv, g_recv_w


def _run_case(idx, E, A, H, cap, x, w, rows, g_result, g_recv, g_recv_w, label):
    log(f"{label}: prepare T={idx.shape[0]} K={idx.shape[1]} E={E} A={A} H={H} cap={cap}")
    run = GpuRun(idx, E, A, H, cap)
    run.prepare()
    p = oracle.prepare(idx, E, A, cap)
    check_prepare(run, p)
    check_all_ops(run, p, x, w, rows, g_result, g_recv, g_recv_w, label=label)
    return run, p


@pytest.mark.parametrize("name,T,H", [
    ("tiny", 256, 512),
    ("mixtral", 1000, 4096),
    ("qwen3", 777, 2048),
    ("dsv3", 501, 7168),
    ("masked", 3001, 1024),
    ("masked_hot", 3001, 1024),
])
def test_parity_reduced(name, T, H):
    cfg = workloads.CONFIGS[name]
    cap = oracle.recv_capacity_worst(T, cfg.K, cfg.E, cfg.A)
    c, r, x, rows, g_result, g_recv, g_recv_w = _inputs(cfg, T, H, cap)
    _run_case(r.topk_idx, c.E, c.A, H, cap, x, r.topk_weights, rows, g_result, g_recv,
              g_recv_w, f"{name}-reduced")


@pytest.mark.parametrize("name", ["mixtral", "qwen3", "dsv3", "masked", "masked_hot"])
def test_parity_full_size(name):
    """Full workload sizes, every element compared. Large payloads are drawn on
    the GPU with a seeded generator and copied to the host for the oracle."""
    _full_size(workloads.CONFIGS[name], name)


def test_parity_dense_routing_past_the_whole_copy_grid():
    """The dsv3 recipe at 12288 tokens: a dense routing whose run copy, sized
    for one step a block, would take more than 128 blocks per CU (5376 a
    stream on 256 CUs), so its grid is capped and every block takes two or
    three steps; every element compared."""
    _full_size(workloads.scaled(workloads.CONFIGS["dsv3"], T=12288), "dsv3-T12288")


def _full_size(cfg, name):
    r = workloads.make_routing(cfg)
    p = oracle.prepare(r.topk_idx, cfg.E, cfg.A,
                       oracle.recv_capacity_worst(cfg.T, cfg.K, cfg.E, cfg.A))
    # the receive buffers at the worst-case capacity, as the benchmark sizes
    # them (for the masked workloads 7.6x the live rows: most of the buffer
    # is tail, which must keep its canary)
    cap = p.cap
    log(f"{name}-full: prepare T={cfg.T} H={cfg.H} cap={cap} total={p.total}")
    run = GpuRun(r.topk_idx, cfg.E, cfg.A, cfg.H, cap)
    run.prepare()
    check_prepare(run, p)
    dev = {"x": workloads.randn_bf16_torch((cfg.T, cfg.H), 11),
           "rows": workloads.randn_bf16_torch((cap, cfg.H), 12),
           "g_result": workloads.randn_bf16_torch((cfg.T, cfg.H), 13),
           "g_recv": workloads.randn_bf16_torch((cap, cfg.H), 14)}
    host = {k: host_bf16(v) for k, v in dev.items()}
    g_recv_w = np.random.default_rng(15).standard_normal(cap, dtype=np.float32)
    check_all_ops(run, p, host["x"], r.topk_weights, host["rows"], host["g_result"],
                  host["g_recv"], g_recv_w, label=f"{name}-full", dev=dev)


def test_masked_local_slice_as_subset_of_global_experts():
    # The masked workload's local slice [0,32) of 256 experts: prepared with
    # E = 32 and with E = 256 on the GPU, every route lands in the same row,
    # the 224 experts past the slice get empty segments, and dispatch writes
    # the same receive buffer.
    cfg = workloads.scaled(workloads.CONFIGS["masked"], T=4096, H=1024)
    r = workloads.make_routing(cfg)
    x = workloads.make_tokens(cfg)
    cap32 = oracle.recv_capacity_worst(cfg.T, cfg.K, 32, cfg.A)
    cap256 = cap32 + 224 * (cfg.A - 1)
    out = {}
    for E, cap in ((32, cap32), (256, cap256)):
        run = GpuRun(r.topk_idx, E, cfg.A, cfg.H, cap)
        run.prepare()
        p = oracle.prepare(r.topk_idx, E, cfg.A, cap)
        check_prepare(run, p)
        recv, recv_w = run.dispatch(dev_bf16(x), dev_f32(r.topk_weights))
        torch.cuda.synchronize()
        out[E] = (run.maps(), run.counts.cpu().numpy(), run.offsets.cpu().numpy(),
                  host_bf16(recv), host_f32(recv_w), p.live)
    m32, c32, o32, rv32, rw32, live = out[32]
    m256, c256, o256, rv256, rw256, live256 = out[256]
    assert live == live256
    assert np.array_equal(m32["slot"], m256["slot"])
    assert np.array_equal(c256[:32], c32) and (c256[32:] == 0).all()
    assert np.array_equal(o256[:33], o32) and (np.diff(o256[32:]) == 0).all()
    assert np.array_equal(rv32[:live], rv256[:live])
    assert np.array_equal(bits32(rw32[:live]), bits32(rw256[:live]))


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------

def _random_payloads(rng, T, H, cap, K):
    x = workloads.randn_bf16(rng, (T, H))
    w = rng.standard_normal((T, K)).astype(np.float32)
    rows = workloads.randn_bf16(rng, (max(cap, 1), H))[:cap]
    g_result = workloads.randn_bf16(rng, (T, H))
    g_recv = workloads.randn_bf16(rng, (max(cap, 1), H))[:cap]
    g_recv_w = rng.standard_normal(cap).astype(np.float32)
    return x, w, rows, g_result, g_recv, g_recv_w


EDGE = [
    # label, T, K, E, A, H, id recipe
    ("no_tokens", 0, 8, 16, 128, 64, "uniform"),
    ("all_masked", 300, 4, 8, 16, 64, "masked"),
    ("one_expert", 500, 1, 1, 8, 64, "uniform"),
    ("no_padding", 700, 2, 8, 1, 128, "uniform"),
    ("generic_k3", 400, 3, 16, 4, 64, "uniform"),
    ("generic_k16", 300, 16, 64, 32, 64, "uniform"),
    ("k64", 100, 64, 128, 8, 64, "uniform"),
    ("h8", 600, 8, 32, 16, 8, "uniform"),
    ("h520_ragged", 333, 4, 16, 16, 520, "uniform"),
    ("many_experts", 900, 8, 2048, 4, 64, "uniform"),
    ("odd_experts", 900, 8, 1000, 128, 64, "uniform"),
    ("big_alignment", 100, 2, 4, 1024, 64, "uniform"),
    ("repeated_ids", 500, 6, 5, 8, 64, "repeats"),
    ("mixed_masks", 1200, 8, 32, 128, 64, "half_masked"),
    # rows of 8 KiB take the interleaved unit order, longer rows the plain one
    ("h4096_interleaved_edge", 300, 8, 64, 16, 4096, "half_masked"),
    ("h4104_plain_ragged", 300, 8, 64, 16, 4104, "half_masked"),
    # routings of up to 4096 routes are prepared by one block in one launch,
    # longer ones by the two-kernel form
    ("prepare_one_block_limit", 512, 8, 64, 16, 64, "half_masked"),
    ("prepare_two_kernels_from", 513, 8, 64, 16, 64, "half_masked"),
    ("prepare_one_block_bad_ids", 700, 5, 37, 8, 64, "bad"),
]


def _edge_ids(rng, T, K, E, recipe):
    if recipe == "masked":
        return np.full((T, K), -1, np.int64)
    if recipe == "repeats":
        return rng.integers(0, E, size=(T, K)).astype(np.int64)
    if recipe == "bad":
        return rng.integers(-3, E + 3, size=(T, K)).astype(np.int64)
    if recipe == "half_masked":
        idx = rng.integers(0, E, size=(T, K))
        return np.where(rng.random((T, K)) < 0.5, -1, idx).astype(np.int64)
    keys = rng.random((T, max(E, K)))
    idx = np.argsort(keys, axis=1)[:, :K]
    return np.where(idx < E, idx, -1).astype(np.int64)


@pytest.mark.parametrize("label,T,K,E,A,H,recipe", EDGE, ids=[e[0] for e in EDGE])
def test_edge_cases(label, T, K, E, A, H, recipe):
    rng = np.random.default_rng(zlib.crc32(label.encode()))
    idx = _edge_ids(rng, T, K, E, recipe)
    cap = T * K + E * (A - 1)
    x, w, rows, g_result, g_recv, g_recv_w = _random_payloads(rng, T, H, cap, K)
    _run_case(idx, E, A, H, cap, x, w, rows, g_result, g_recv, g_recv_w, label)


def test_bad_expert_ids_flagged_and_dropped():
    rng = np.random.default_rng(1)
    T, K, E, A, H = 400, 4, 16, 8, 64
    idx = rng.integers(0, E, size=(T, K)).astype(np.int64)
    idx[5, 1] = E          # out of range (the num_experts sentinel is not a mask here)
    idx[17, 0] = -2
    idx[300, 3] = 1 << 40
    cap = T * K + E * (A - 1)
    x, w, rows, g_result, g_recv, g_recv_w = _random_payloads(rng, T, H, cap, K)
    run, p = _run_case(idx, E, A, H, cap, x, w, rows, g_result, g_recv, g_recv_w, "bad_ids")
    assert p.status == oracle.STATUS_BAD_EXPERT


@pytest.mark.parametrize("cap_frac", [0.5, 0.0])
def test_overflow_drops_routes_past_capacity(cap_frac):
    rng = np.random.default_rng(2)
    T, K, E, A, H = 600, 8, 32, 16, 64
    idx = _edge_ids(rng, T, K, E, "uniform")
    worst = T * K + E * (A - 1)
    cap = int(worst * cap_frac)
    x, w, rows, g_result, g_recv, g_recv_w = _random_payloads(rng, T, H, cap, K)
    run, p = _run_case(idx, E, A, H, cap, x, w, rows, g_result, g_recv, g_recv_w,
                       f"overflow-{cap_frac}")
    assert p.status == oracle.STATUS_OVERFLOW


def test_special_values_in_combine():
    specials = np.array([0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x0001, 0x8001,
                         0x007F, 0x7F7F, 0xFF7F, 0x3F80, 0xBF80, 0x0080, 0x4B80, 0xCB80],
                        np.uint16)
    rng = np.random.default_rng(3)
    T, K, E, A, H = 512, 8, 8, 4, 256
    idx = rng.integers(-1, E, size=(T, K)).astype(np.int64)
    cap = T * K + E * (A - 1)
    rows = rng.choice(specials, size=(cap, H))
    x, w, _, g_result, _, g_recv_w = _random_payloads(rng, T, H, cap, K)
    g_recv = rng.choice(specials, size=(cap, H))
    _run_case(idx, E, A, H, cap, x, w, rows, g_result, g_recv, g_recv_w, "specials")


def test_null_weight_gradients_and_outputs():
    rng = np.random.default_rng(4)
    T, K, E, A, H = 300, 4, 8, 16, 64
    idx = _edge_ids(rng, T, K, E, "uniform")
    cap = T * K + E * (A - 1)
    x, w, rows, g_result, g_recv, g_recv_w = _random_payloads(rng, T, H, cap, K)
    run = GpuRun(idx, E, A, H, cap)
    run.prepare(with_offsets=False)
    p = oracle.prepare(idx, E, A, cap)
    # no g_recv_topk_weights: the weight gradient is +0 everywhere
    gt, gw = run.dispatch_bwd(dev_bf16(g_recv), None)
    assert (bits32(host_f32(gw)) == 0).all()
    assert np.array_equal(host_bf16(gt), oracle.combine(p, g_recv))
    # no grad_topk_weights output: only the token gradient is written
    gt2, _ = run.dispatch_bwd(dev_bf16(g_recv), dev_f32(g_recv_w), want_w=False)
    assert np.array_equal(host_bf16(gt2), host_bf16(gt))
    # dispatch without weights
    recv, _ = run.dispatch(dev_bf16(x), None)
    o_recv, _ = oracle.dispatch(p, x, None, recv_init=np.full((cap, H), CANARY_BF16, np.uint16))
    assert np.array_equal(host_bf16(recv), o_recv)
    # expert_offsets was not requested: the buffer keeps its fill value
    assert (run.offsets.cpu().numpy() == -5).all()


# ---------------------------------------------------------------------------
# properties
# ---------------------------------------------------------------------------

def test_adjoint_maps_share_kernels_bitwise():
    cfg = workloads.CONFIGS["dsv3"]
    T, H = 700, 1024
    cap = oracle.recv_capacity_worst(T, cfg.K, cfg.E, cfg.A)
    c, r, x, rows, g_result, g_recv, g_recv_w = _inputs(cfg, T, H, cap, seed=3)
    run = GpuRun(r.topk_idx, c.E, c.A, H, cap)
    run.prepare()
    g = dev_bf16(g_result)
    recv, _ = run.dispatch(g, None)
    gb = run.combine_bwd(g)
    assert torch.equal(recv.view(torch.int16), gb.view(torch.int16))
    G = dev_bf16(g_recv)
    comb = run.combine(G)
    gt, _ = run.dispatch_bwd(G, None)
    assert torch.equal(comb.view(torch.int16), gt.view(torch.int16))


def test_identity_round_trip_on_gpu():
    cfg = workloads.CONFIGS["tiny"]
    r = workloads.make_routing(cfg)
    x = workloads.make_tokens(cfg)
    cap = oracle.recv_capacity_worst(cfg.T, cfg.K, cfg.E, cfg.A)
    run = GpuRun(r.topk_idx, cfg.E, cfg.A, cfg.H, cap)
    run.prepare()
    recv, _ = run.dispatch(dev_bf16(x), None)
    out = run.combine(recv)
    want = (torch.from_numpy(workloads.bf16_to_f32(x)) * 2).to(torch.bfloat16)
    assert torch.equal(out.cpu().view(torch.int16), want.view(torch.int16))


def test_repeatable_and_interleaved_handles():
    cfg = workloads.CONFIGS["qwen3"]
    T, H = 1500, 512
    cap = oracle.recv_capacity_worst(T, cfg.K, cfg.E, cfg.A)
    c1, r1, x1, rows1, *_ = _inputs(cfg, T, H, cap, seed=1)
    c2, r2, x2, rows2, *_ = _inputs(cfg, T, H, cap, seed=2)
    a = GpuRun(r1.topk_idx, c1.E, c1.A, H, cap)
    b = GpuRun(r2.topk_idx, c2.E, c2.A, H, cap)
    a.prepare()
    b.prepare()                      # both handles live at once
    xa, xb = dev_bf16(x1), dev_bf16(x2)
    ra, rb = dev_bf16(rows1), dev_bf16(rows2)
    first = [a.dispatch(xa, None)[0], b.dispatch(xb, None)[0], a.combine(ra), b.combine(rb)]
    for _ in range(3):
        a.prepare()
        again = [a.dispatch(xa, None)[0], b.dispatch(xb, None)[0], a.combine(ra),
                 b.combine(rb)]
        for f, g in zip(first, again):
            assert torch.equal(f.view(torch.int16), g.view(torch.int16))
    pa = oracle.prepare(r1.topk_idx, c1.E, c1.A, cap)
    pb = oracle.prepare(r2.topk_idx, c2.E, c2.A, cap)
    assert np.array_equal(host_bf16(first[2]), oracle.combine(pa, rows1))
    assert np.array_equal(host_bf16(first[3]), oracle.combine(pb, rows2))


def test_non_default_stream():
    cfg = workloads.CONFIGS["mixtral"]
    T, H = 2000, 512
    cap = oracle.recv_capacity_worst(T, cfg.K, cfg.E, cfg.A)
    c, r, x, rows, g_result, g_recv, g_recv_w = _inputs(cfg, T, H, cap, seed=4)
    s = torch.cuda.Stream()
    xd, rd = dev_bf16(x), dev_bf16(rows)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        run = GpuRun(r.topk_idx, c.E, c.A, H, cap, stream=s)
        run.prepare()
        recv, recv_w = run.dispatch(xd, dev_f32(r.topk_weights))
        out = run.combine(rd)
    s.synchronize()
    p = oracle.prepare(r.topk_idx, c.E, c.A, cap)
    o_recv, _ = oracle.dispatch(p, x, r.topk_weights,
                                recv_init=np.full((cap, H), CANARY_BF16, np.uint16))
    assert np.array_equal(host_bf16(recv), o_recv)
    assert np.array_equal(host_bf16(out), oracle.combine(p, rows))


def test_layout_mismatch_is_flagged_and_writes_nothing():
    import combine_ep_prepare_amd as ep
    rng = np.random.default_rng(6)
    T, K, E, A, H = 256, 4, 8, 16, 64
    idx = _edge_ids(rng, T, K, E, "uniform")
    cap = T * K + E * (A - 1)
    run = GpuRun(idx, E, A, H, cap)
    run.prepare()
    assert run.status() == 0
    # same handle, a different alignment: the payload op refuses on the device
    other = ep.Layout(T, K, E, A * 2, H, cap)
    assert ep.handle_mem_size(other) <= run.handle.numel()
    x = dev_bf16(workloads.randn_bf16(rng, (T, H)))
    from gpu_harness import _fill_bf16
    recv = _fill_bf16(cap, H)
    ep.dispatch(other, run.handle, x, None, recv, None)
    assert run.status() == ep.STATUS_LAYOUT
    assert (host_bf16(recv) == CANARY_BF16).all()
    # prepare resets the status word
    run.prepare()
    assert run.status() == 0
    # a handle that was never prepared
    fresh = torch.zeros_like(run.handle)
    recv = _fill_bf16(cap, H)
    ep.combine_bwd(run.layout, fresh, x, recv)
    torch.cuda.synchronize()
    assert ep.read_status(fresh) == ep.STATUS_LAYOUT
    assert (host_bf16(recv) == CANARY_BF16).all()
