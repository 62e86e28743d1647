"""GPU parity of the fp16 and fp32 payload paths and of the no-pad-fill policy.

Every op runs through the C ABI with the layout's payload type and pad
policy and is compared with the oracle bit for bit (the weighted backward's
weight gradient within its summation bound), outputs pre-filled with a
canary so that rows that must stay unwritten are checked too.
"""
import zlib

import numpy as np
import pytest
import torch

import combine_ep_prepare_amd as ep
import oracle
import workloads
from gpu_harness import log, wbwd_gamma

pytestmark = pytest.mark.gpu

TORCH = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}
NP = {"bf16": np.uint16, "fp16": np.uint16, "fp32": np.float32}
CANARY = {"bf16": 0xBEEF, "fp16": 0xBEEF, "fp32": np.float32(-1234.5)}
CANARY_W = np.float32(-1234.5)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build()


def dev(a, dt):
    a = np.ascontiguousarray(a, dtype=NP[dt])
    if dt == "fp32":
        return torch.from_numpy(a).cuda()
    return torch.from_numpy(a.view(np.int16)).cuda().view(TORCH[dt])


def host(t, dt):
    if dt == "fp32":
        return t.cpu().numpy()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def bits(a):
    a = np.asarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16)


def canary_rows(n, H, dt):
    if dt == "fp32":
        return torch.full((n, H), float(CANARY[dt]), dtype=torch.float32, device="cuda")
    t = torch.empty((n, H), dtype=torch.int16, device="cuda")
    t.fill_(np.array([CANARY[dt]], np.uint16).view(np.int16)[0].item())
    return t.view(TORCH[dt])


def canary_host(n, H, dt):
    return np.full((n, H), CANARY[dt], NP[dt])


def canary_w(n):
    return torch.full((n,), float(CANARY_W), dtype=torch.float32, device="cuda")


def payload(rng, shape, dt, specials=False):
    v = rng.standard_normal(shape).astype(np.float32)
    if dt == "bf16":
        out = workloads._bf16_bits(v)
    elif dt == "fp16":
        out = (v * 4).astype(np.float16).view(np.uint16)
    else:
        out = v
    if specials:
        sp = {"bf16": np.array([0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0x0001, 0x7F7F],
                               np.uint16),
              "fp16": np.array([0x0000, 0x8000, 0x7C00, 0xFC00, 0x7E00, 0x0001, 0x8001,
                                0x03FF, 0x7BFF, 0x6800], np.uint16),
              "fp32": np.array([0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000,
                                0x00000001, 0x807FFFFF, 0x7F7FFFFF], np.uint32
                               ).view(np.float32)}[dt]
        out = out.copy()
        m = rng.random(shape) < 0.1
        out[m] = rng.choice(sp, size=int(m.sum()))
    return out


def run_case(label, idx, E, A, H, cap, dt, fill_pads, rng, specials=False,
             zero_tail=False):
    T, K = idx.shape
    log(f"dtypes {label}: dt={dt} fill_pads={fill_pads} zero_tail={zero_tail} "
        f"T={T} K={K} E={E} A={A} H={H} cap={cap}")
    L = ep.Layout(T, K, E, A, H, cap, dtype=dt, fill_pads=fill_pads, zero_tail=zero_tail)
    handle = ep.new_handle(L)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    ep.prepare(L, torch.from_numpy(idx).cuda(), counts, handle)
    p = oracle.prepare(idx, E, A, cap)
    live = p.live
    x = payload(rng, (T, H), dt, specials)
    w = rng.standard_normal((T, K)).astype(np.float32)
    Y = payload(rng, (cap, H), dt, specials)
    g = payload(rng, (T, H), dt, specials)
    G = payload(rng, (cap, H), dt, specials)
    Gw = rng.standard_normal(cap).astype(np.float32)
    rw = rng.standard_normal(cap).astype(np.float32)
    xd, Yd, gd, Gd = dev(x, dt), dev(Y, dt), dev(g, dt), dev(G, dt)
    kw = dict(dtype=dt, fill_pads=fill_pads, zero_tail=zero_tail)

    # dispatch
    recv, recv_w = canary_rows(cap, H, dt), canary_w(cap)
    ep.dispatch(L, handle, xd, torch.from_numpy(w).cuda(), recv, recv_w)
    o_recv, o_recv_w = oracle.dispatch(p, x, w, recv_init=canary_host(cap, H, dt),
                                       recv_w_init=np.full(cap, CANARY_W, np.float32), **kw)
    assert np.array_equal(bits(host(recv, dt)), bits(o_recv)), f"{label} dispatch"
    assert np.array_equal(bits(recv_w.cpu().numpy()), bits(o_recv_w)), f"{label} dispatch w"
    # combine
    out = canary_rows(T, H, dt)
    ep.combine(L, handle, Yd, out)
    assert np.array_equal(bits(host(out, dt)), bits(oracle.combine(p, Y, dtype=dt))), \
        f"{label} combine"
    # combine_bwd
    gx = canary_rows(cap, H, dt)
    ep.combine_bwd(L, handle, gd, gx)
    assert np.array_equal(bits(host(gx, dt)),
                          bits(oracle.combine_bwd(p, g, init=canary_host(cap, H, dt), **kw))), \
        f"{label} combine_bwd"
    # dispatch_bwd
    gt, gw = canary_rows(T, H, dt), canary_w(T * K).view(T, K)
    ep.dispatch_bwd(L, handle, Gd, torch.from_numpy(Gw).cuda(), gt, gw)
    o_gt, o_gw = oracle.dispatch_bwd(p, G, Gw, dtype=dt)
    assert np.array_equal(bits(host(gt, dt)), bits(o_gt)), f"{label} dispatch_bwd"
    assert np.array_equal(bits(gw.cpu().numpy()), bits(o_gw)), f"{label} dispatch_bwd w"
    # weighted combine
    rwd = torch.from_numpy(rw).cuda()
    outw = canary_rows(T, H, dt)
    ep.combine_weighted(L, handle, Yd, rwd, outw)
    assert np.array_equal(bits(host(outw, dt)),
                          bits(oracle.combine_weighted(p, Y, rw, dtype=dt))), \
        f"{label} combine_weighted"
    # its backward (finite inputs only for the dot product bound)
    if not specials:
        gr, gwr = canary_rows(cap, H, dt), canary_w(cap)
        ep.combine_weighted_bwd(L, handle, gd, Yd, rwd, gr, gwr)
        o_gr, o_gwr, o_abs = oracle.combine_weighted_bwd(
            p, g, Y, rw, init=canary_host(cap, H, dt), **kw)
        assert np.array_equal(bits(host(gr, dt)), bits(o_gr)), f"{label} weighted_bwd rows"
        got = gwr.cpu().numpy().astype(np.float64)
        pad = np.zeros(cap, bool)
        pad[:live] = p.row_src[:live] < 0
        tok = np.zeros(cap, bool)
        tok[:live] = ~pad[:live]
        err = np.abs(got[tok] - o_gwr[tok])
        assert (err <= wbwd_gamma(H, dt) * o_abs[tok] + 1e-45).all(), f"{label} weighted_bwd w"
        want_pad = 0.0 if fill_pads else float(CANARY_W)
        assert (got[pad] == want_pad).all()
        assert (got[live:] == (0.0 if zero_tail else float(CANARY_W))).all()
    assert ep.read_status(handle) == p.status


CONFIG_CASES = [("tiny", 256, 512), ("qwen3", 700, 2048), ("dsv3", 300, 7168),
                ("masked_hot", 2500, 1024)]


@pytest.mark.parametrize("dt", ["fp16", "fp32"])
@pytest.mark.parametrize("name,T,H", CONFIG_CASES)
def test_payload_type_parity(dt, name, T, H):
    c = workloads.scaled(workloads.CONFIGS[name], T=T, H=H)
    r = workloads.make_routing(c)
    cap = oracle.recv_capacity_worst(T, c.K, c.E, c.A)
    run_case(name, r.topk_idx, c.E, c.A, H, cap, dt, True,
             np.random.default_rng(zlib.crc32(f"{name}{dt}".encode())))


@pytest.mark.parametrize("dt", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("name,T,H", [("dsv3", 300, 1024), ("qwen3", 500, 512),
                                     ("dsv3", 200, 4104)])
def test_no_pad_fill_parity(dt, name, T, H):
    c = workloads.scaled(workloads.CONFIGS[name], T=T, H=H)
    r = workloads.make_routing(c)
    cap = oracle.recv_capacity_worst(T, c.K, c.E, c.A)
    run_case(name + "-nopad", r.topk_idx, c.E, c.A, H, cap, dt, False,
             np.random.default_rng(zlib.crc32(f"{name}{dt}nopad".encode())))


@pytest.mark.parametrize("dt", ["fp16", "fp32"])
@pytest.mark.parametrize("label,T,K,E,A,H,shrink", [
    ("generic_k3", 300, 3, 16, 4, 64, False), ("generic_k12", 150, 12, 40, 8, 136, False),
    ("overflow", 400, 8, 32, 16, 72, True), ("ragged_cols", 257, 2, 5, 3, 1032, False),
    ("ragged_long_rows", 157, 6, 9, 5, 2056, False)])
def test_payload_type_edge_cases(dt, label, T, K, E, A, H, shrink):
    rng = np.random.default_rng(zlib.crc32(f"{label}{dt}".encode()))
    idx = np.argsort(rng.random((T, max(E, K))), axis=1)[:, :K]
    idx = np.where(idx < E, idx, -1).astype(np.int64)
    idx[rng.random((T, K)) < 0.25] = -1
    cap = T * K + E * (A - 1)
    if shrink:
        cap //= 3
    run_case(label, idx, E, A, H, cap, dt, True, rng)
    run_case(label + "-nopad", idx, E, A, H, cap, dt, False, rng)


@pytest.mark.parametrize("dt", ["fp16", "fp32"])
def test_payload_type_special_values(dt):
    c = workloads.scaled(workloads.CONFIGS["qwen3"], T=400, H=256)
    r = workloads.make_routing(c)
    cap = oracle.recv_capacity_worst(c.T, c.K, c.E, c.A)
    run_case("specials", r.topk_idx, c.E, c.A, c.H, cap, dt, True,
             np.random.default_rng(77), specials=True)


@pytest.mark.parametrize("dt,prep", [("fp16", "fp16"), ("fp32", "fp32"), ("fp32", "bf16")])
def test_full_size_dsv3_dispatch_combine(dt, prep):
    # the DeepSeek-V3-shaped workload at full size: dispatch, combine and
    # combine_bwd, from a handle prepared for the same payload type (run
    # chunks sized for its rows, as the benchmark prepares its fp32 ops) and
    # from one prepared for bf16 rows (chunks twice as many fp32 bytes)
    cfg = workloads.CONFIGS["dsv3"]
    r = workloads.make_routing(cfg)
    T, K, E, A, H = cfg.T, cfg.K, cfg.E, cfg.A, cfg.H
    cap = oracle.recv_capacity_worst(T, K, E, A)
    log(f"dtypes full dsv3 {dt}, prepared for {prep}: T={T} H={H} cap={cap}")
    L = ep.Layout(T, K, E, A, H, cap, dtype=dt)
    handle = ep.new_handle(L)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    ep.prepare(ep.Layout(T, K, E, A, H, cap, dtype=prep), torch.from_numpy(r.topk_idx).cuda(),
               counts, handle)
    p = oracle.prepare(r.topk_idx, E, A, cap)
    rng = np.random.default_rng(5)
    x = payload(rng, (T, H), dt)
    recv = canary_rows(cap, H, dt)
    ep.dispatch(L, handle, dev(x, dt), None, recv, None)
    got = host(recv, dt)
    want, _ = oracle.dispatch(p, x, None, recv_init=canary_host(cap, H, dt), dtype=dt)
    assert np.array_equal(bits(got), bits(want))
    del recv, got, want
    Y = payload(rng, (cap, H), dt)
    out = canary_rows(T, H, dt)
    ep.combine(L, handle, dev(Y, dt), out)
    assert np.array_equal(bits(host(out, dt)), bits(oracle.combine(p, Y, dtype=dt)))
    del Y, out
    g = payload(rng, (T, H), dt)
    gx = canary_rows(cap, H, dt)
    ep.combine_bwd(L, handle, dev(g, dt), gx)
    want = oracle.combine_bwd(p, g, init=canary_host(cap, H, dt), dtype=dt)
    assert np.array_equal(bits(host(gx, dt)), bits(want))


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
@pytest.mark.parametrize("fill_pads", [True, False])
@pytest.mark.parametrize("name,T,H", [("masked", 1500, 512), ("dsv3", 200, 1024),
                                     ("mixtral", 3000, 256)])
def test_zero_tail_parity(dt, fill_pads, name, T, H):
    # the tail policy: rows past the live total of every expert-major output
    # are zeros (canaries elsewhere where the pad policy leaves rows alone),
    # on both copy paths, with and without the pad fill
    c = workloads.scaled(workloads.CONFIGS[name], T=T, H=H)
    r = workloads.make_routing(c)
    cap = oracle.recv_capacity_worst(T, c.K, c.E, c.A)
    run_case(f"{name}-tail", r.topk_idx, c.E, c.A, H, cap, dt, fill_pads,
             np.random.default_rng(zlib.crc32(f"{name}{dt}{fill_pads}".encode())),
             zero_tail=True)


def test_zero_tail_without_tokens():
    # T = 0: every row is past the live total (which is 0)
    L = ep.Layout(0, 4, 8, 16, 64, 300, zero_tail=True)
    handle = ep.new_handle(L)
    counts = torch.empty(8, dtype=torch.int32, device="cuda")
    ep.prepare(L, torch.empty(0, 4, dtype=torch.int64, device="cuda"), counts, handle)
    recv, recv_w = canary_rows(300, 64, "bf16"), canary_w(300)
    ep.dispatch(L, handle, torch.empty(0, 64, dtype=torch.bfloat16, device="cuda"),
                torch.empty(0, 4, device="cuda"), recv, recv_w)
    gx = canary_rows(300, 64, "bf16")
    ep.combine_bwd(L, handle, torch.empty(0, 64, dtype=torch.bfloat16, device="cuda"), gx)
    torch.cuda.synchronize()
    assert (host(recv, "bf16") == 0).all() and (recv_w.cpu().numpy() == 0).all()
    assert (host(gx, "bf16") == 0).all()
    assert ep.read_status(handle) == 0
