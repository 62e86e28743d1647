"""GPU parity of the weighted combine and its backward.

Forward and the row gradient are bit-exact against the oracle. The weight
gradient is a dot product over H whose order the method does not fix; it is
compared with the oracle's double-precision dot within the summation error
bound of the kernel's fixed order: each 64-lane piece of a row (P =
ceil(V/64) of them, V = H/8 16-byte vectors) is a per-lane chain of 8 fused
multiply-adds, then 6 butterfly adds over the lanes, and the P partials are
summed in piece order, so |got - exact| <= gamma_n * sum_h |g_h y_h| with
n = 8 + P + 5 and gamma_n = n u / (1 - n u), u = 2^-24. It must also be
bit-identical from run to run.
"""
import zlib

import numpy as np
import pytest
import torch

import combine_ep_prepare_amd as ep
import oracle
import workloads
from gpu_harness import (CANARY_BF16, wbwd_gamma, CANARY_F32, GpuRun, _fill_bf16, _fill_f32, bits32,
                         dev_bf16, dev_f32, host_bf16, host_f32, log)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build()


def _case(label, idx, E, A, H, cap, rng):
    T, K = idx.shape
    log(f"weighted {label}: T={T} K={K} E={E} A={A} H={H} cap={cap}")
    run = GpuRun(idx, E, A, H, cap)
    run.prepare()
    p = oracle.prepare(idx, E, A, cap)
    Y = workloads.randn_bf16(rng, (max(cap, 1), H))[:cap]
    w = rng.standard_normal(cap).astype(np.float32)
    g = workloads.randn_bf16(rng, (T, H))
    Yd, wd, gd = dev_bf16(Y), dev_f32(w), dev_bf16(g)
    # forward
    out = _fill_bf16(T, H)
    ep.combine_weighted(run.layout, run.handle, Yd, wd, out)
    assert np.array_equal(host_bf16(out), oracle.combine_weighted(p, Y, w)), label
    # backward, both outputs
    gr = _fill_bf16(cap, H)
    gw = _fill_f32(cap)
    ep.combine_weighted_bwd(run.layout, run.handle, gd, Yd, wd, gr, gw)
    o_gr, o_gw, o_abs = oracle.combine_weighted_bwd(
        p, g, Y, w, init=np.full((cap, H), CANARY_BF16, np.uint16))
    assert np.array_equal(host_bf16(gr), o_gr), label
    live = p.live
    got = host_f32(gw).astype(np.float64)
    assert (got[live:] == float(CANARY_F32)).all(), label          # untouched past live
    err = np.abs(got[:live] - o_gw[:live])
    bound = wbwd_gamma(H) * o_abs[:live] + 1e-45
    assert (err <= bound).all(), (label, float((err / np.maximum(bound, 1e-300)).max()))
    pad = p.row_src[:live] < 0
    assert (bits32(host_f32(gw))[:live][pad] == 0).all()
    # run to run: bit-identical
    gw2 = _fill_f32(cap)
    ep.combine_weighted_bwd(run.layout, run.handle, gd, Yd, wd, gr, gw2)
    assert np.array_equal(bits32(host_f32(gw)), bits32(host_f32(gw2))), label
    # row gradient only (no expert_out needed)
    gr3 = _fill_bf16(cap, H)
    ep.combine_weighted_bwd(run.layout, run.handle, gd, None, wd, gr3, None)
    assert np.array_equal(host_bf16(gr3), o_gr), label


@pytest.mark.parametrize("name,T,H", [("tiny", 256, 512), ("mixtral", 900, 4096),
                                      ("qwen3", 600, 2048), ("dsv3", 400, 7168),
                                      ("masked_hot", 3000, 1024)])
def test_weighted_parity(name, T, H):
    cfg = workloads.CONFIGS[name]
    c = workloads.scaled(cfg, T=T, H=H)
    r = workloads.make_routing(c)
    cap = oracle.recv_capacity_worst(T, c.K, c.E, c.A)
    _case(name, r.topk_idx, c.E, c.A, H, cap, np.random.default_rng(zlib.crc32(name.encode())))


@pytest.mark.parametrize("label,T,K,E,A,H", [("generic_k3", 300, 3, 16, 4, 64),
                                             ("generic_k12", 200, 12, 40, 8, 136),
                                             ("one_route", 333, 1, 8, 16, 520),
                                             ("overflow", 500, 8, 32, 16, 64),
                                             ("wide_rows", 96, 4, 16, 4, 20488)])
def test_weighted_edge_cases(label, T, K, E, A, H):
    rng = np.random.default_rng(zlib.crc32(label.encode()))
    keys = rng.random((T, max(E, K)))
    idx = np.argsort(keys, axis=1)[:, :K]
    idx = np.where(idx < E, idx, -1).astype(np.int64)
    idx[rng.random((T, K)) < 0.3] = -1
    cap = T * K + E * (A - 1)
    if label == "overflow":
        cap //= 3
    _case(label, idx, E, A, H, cap, rng)


@pytest.mark.parametrize("label,masked", [("sparse_rows", 0.85), ("dense_lists", 0.0)])
def test_weighted_both_walks(label, masked):
    """The backward walks the received rows in order when fewer than half of
    the routes hold a row, else the run lists: the same routing shape on
    either side, every output checked."""
    T, K, E, A, H = 1500, 8, 48, 8, 1032
    rng = np.random.default_rng(zlib.crc32(label.encode()))
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int64)
    idx[rng.random((T, K)) < masked] = -1
    _case(label, idx, E, A, H, T * K + E * (A - 1), rng)


def test_weighted_sparse_rows_in_several_rounds():
    """The hot-expert recipe at 20000 tokens and H = 7168: the received rows
    (about 37000 of them) outnumber what one round of the capped grid takes
    (32768 on 256 CUs), so blocks walk rows in two rounds."""
    cfg = workloads.scaled(workloads.CONFIGS["masked_hot"], T=20000)
    r = workloads.make_routing(cfg)
    p = oracle.prepare(r.topk_idx, cfg.E, cfg.A,
                       oracle.recv_capacity_worst(cfg.T, cfg.K, cfg.E, cfg.A))
    cap = (p.total + 4095) // 4096 * 4096
    _case("masked_hot-T20000", r.topk_idx, cfg.E, cfg.A, cfg.H, cap,
          np.random.default_rng(34))


def test_weighted_full_size_dsv3():
    cfg = workloads.CONFIGS["dsv3"]
    r = workloads.make_routing(cfg)
    cap = oracle.recv_capacity_worst(cfg.T, cfg.K, cfg.E, cfg.A)
    _case("dsv3-full", r.topk_idx, cfg.E, cfg.A, cfg.H, cap, np.random.default_rng(33))
