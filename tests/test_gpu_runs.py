"""GPU parity of the run-entry copy that dispatch and combine_bwd use for every
routing, across the run-entry layouts prepare can build.

Prepare cuts the routes into chunks of 1, 2 or 4 units of 512 routes, sized
from its own layout's payload row (so that a chunk's token rows fit an XCD's
L2), and lays each of the eight streams' chunks out as one list. The payload
ops read those lists whatever their own payload type. Every case here checks
the lists against their definition (gpu_harness.check_run_entries) and every
op against the oracle bit for bit, canaries included: routings prepared for
another row size than the payload ops use, unit and stream boundaries, the
one-block and two-kernel prepares, masked routes, bad ids, overflow, long
rows, payload types and pad policies.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_harness import GpuRun, check_all_ops, check_prepare, log
from test_gpu_dtypes import run_case
from test_gpu_parity import EDGE, _edge_ids, _inputs, _random_payloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build()


def _runs_case(idx, E, A, H, cap, x, w, rows, g_result, g_recv, g_recv_w, label,
               prepare_dtype="bf16"):
    log(f"{label}: prepare for {prepare_dtype} T={idx.shape[0]} K={idx.shape[1]} E={E} "
        f"A={A} H={H} cap={cap}")
    run = GpuRun(idx, E, A, H, cap, prepare_dtype=prepare_dtype)
    run.prepare()
    p = oracle.prepare(idx, E, A, cap)
    check_prepare(run, p)          # includes the run entries
    check_all_ops(run, p, x, w, rows, g_result, g_recv, g_recv_w, label=label)
    return p


@pytest.mark.parametrize("name,T,H", [
    ("tiny", 256, 512), ("mixtral", 1000, 4096), ("qwen3", 777, 2048), ("dsv3", 501, 7168),
    ("dsv3", 2049, 1032), ("masked", 3001, 1024), ("masked_hot", 3001, 1024),
])
def test_runs_prepared_for_fp32_rows(name, T, H):
    """Prepared with the fp32 layout (chunks sized for rows twice as long),
    used with bf16 payloads."""
    cfg = workloads.CONFIGS[name]
    cap = oracle.recv_capacity_worst(T, cfg.K, cfg.E, cfg.A)
    c, r, x, rows, g_result, g_recv, g_recv_w = _inputs(cfg, T, H, cap, seed=3)
    _runs_case(r.topk_idx, c.E, c.A, H, cap, x, r.topk_weights, rows, g_result, g_recv,
               g_recv_w, f"{name}-prep-fp32", prepare_dtype="fp32")


@pytest.mark.parametrize("label,T,K,E,A,H,recipe", EDGE, ids=[e[0] for e in EDGE])
def test_runs_edge_cases_prepared_for_fp32_rows(label, T, K, E, A, H, recipe):
    rng = np.random.default_rng(zlib.crc32(("runs" + label).encode()))
    idx = _edge_ids(rng, T, K, E, recipe)
    cap = T * K + E * (A - 1)
    x, w, rows, g_result, g_recv, g_recv_w = _random_payloads(rng, T, H, cap, K)
    _runs_case(idx, E, A, H, cap, x, w, rows, g_result, g_recv, g_recv_w, label + "-runs",
               prepare_dtype="fp32")


@pytest.mark.parametrize("T", [1, 127, 128, 129, 1023, 1024, 1025, 4095, 4097, 8192, 8320])
def test_runs_unit_and_stream_boundaries(T):
    """Route counts (4 per token) around the 512-route units, the 4096-route
    cutover between the one-block and the two-kernel prepare, and chunks of 1,
    2 and 4 units dealt to eight streams (one or more chunks each)."""
    rng = np.random.default_rng(T)
    K, E, A, H = 4, 24, 8, 72
    idx = _edge_ids(rng, T, K, E, "uniform")
    idx[rng.random((T, K)) < 0.2] = -1
    cap = T * K + E * (A - 1)
    x, w, rows, g_result, g_recv, g_recv_w = _random_payloads(rng, T, H, cap, K)
    for prep in ("bf16", "fp32"):
        _runs_case(idx, E, A, H, cap, x, w, rows, g_result, g_recv, g_recv_w,
                   f"units-T{T}", prepare_dtype=prep)


@pytest.mark.parametrize("cap_frac", [0.5, 0.0])
def test_runs_overflow(cap_frac):
    """Routes dropped past the capacity leave empty entries in their lists."""
    rng = np.random.default_rng(12)
    T, K, E, A, H = 1600, 8, 32, 16, 64
    idx = _edge_ids(rng, T, K, E, "uniform")
    cap = int((T * K + E * (A - 1)) * cap_frac)
    x, w, rows, g_result, g_recv, g_recv_w = _random_payloads(rng, T, H, cap, K)
    p = _runs_case(idx, E, A, H, cap, x, w, rows, g_result, g_recv, g_recv_w,
                   f"runs-overflow-{cap_frac}")
    assert p.status == oracle.STATUS_OVERFLOW


@pytest.mark.parametrize("dt", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("fill_pads", [True, False])
@pytest.mark.parametrize("name,T,H", [("dsv3", 300, 1024), ("qwen3", 500, 512),
                                     ("mixtral", 400, 264)])
def test_runs_payload_types_and_pad_policy(dt, fill_pads, name, T, H):
    c = workloads.scaled(workloads.CONFIGS[name], T=T, H=H)
    r = workloads.make_routing(c)
    cap = oracle.recv_capacity_worst(T, c.K, c.E, c.A)
    run_case(name + "-runs", r.topk_idx, c.E, c.A, H, cap, dt, fill_pads,
             np.random.default_rng(zlib.crc32(f"{name}{dt}{fill_pads}runs".encode())))


@pytest.mark.parametrize("fill_pads", [True, False])
@pytest.mark.parametrize("T,H", [(1, 6144), (9, 6152), (300, 6144), (2049, 6152)])
def test_runs_long_rows(T, H, fill_pads):
    """Rows of 12 KiB and more, with and without the pad fill: 6144 is exactly
    12 pieces of 1 KiB, 6152 has a ragged 13th; token counts around the unit
    boundaries."""
    rng = np.random.default_rng(zlib.crc32(f"long{T}-{H}-{fill_pads}".encode()))
    K, E, A = 8, 64, 16
    idx = _edge_ids(rng, T, K, E, "uniform")
    cap = T * K + E * (A - 1)
    run_case(f"long-T{T}-H{H}", idx, E, A, H, cap, "bf16", fill_pads, rng)
