"""GPU parity of the dense-routing path (EP_LAYOUT_DENSE_ROUTING).

With the flag, dispatch and combine_bwd copy rows over the run entries that
prepare builds (chunks of tokens, rows in ascending order) instead of
scattering token by token. The flag is a speed hint: every result must still
equal the oracle's bit for bit, canaries included, for dense routings (what
the flag states) and for routings that break the statement (masked routes,
bad ids, overflow), which the path must still handle correctly.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_harness import GpuRun, check_all_ops, check_prepare, check_run_entries, host_bf16, log
from test_gpu_dtypes import run_case
from test_gpu_parity import EDGE, _edge_ids, _inputs, _random_payloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build()


def _dense_case(idx, E, A, H, cap, x, w, rows, g_result, g_recv, g_recv_w, label, dev=None):
    log(f"{label}: dense prepare T={idx.shape[0]} K={idx.shape[1]} E={E} A={A} H={H} cap={cap}")
    run = GpuRun(idx, E, A, H, cap, dense=True)
    run.prepare()
    p = oracle.prepare(idx, E, A, cap)
    check_prepare(run, p)
    if idx.shape[0] > 0:
        check_run_entries(run.maps(), p.slot, idx, E)
    check_all_ops(run, p, x, w, rows, g_result, g_recv, g_recv_w, label=label, dev=dev)
    return p


@pytest.mark.parametrize("name", ["mixtral", "qwen3", "dsv3"])
def test_dense_full_size(name):
    """The configurations the benchmark times with the flag, every element."""
    cfg = workloads.CONFIGS[name]
    r = workloads.make_routing(cfg)
    assert (r.topk_idx >= 0).all()
    cap = oracle.recv_capacity_worst(cfg.T, cfg.K, cfg.E, cfg.A)
    dev = {"x": workloads.randn_bf16_torch((cfg.T, cfg.H), 21),
           "rows": workloads.randn_bf16_torch((cap, cfg.H), 22),
           "g_result": workloads.randn_bf16_torch((cfg.T, cfg.H), 23),
           "g_recv": workloads.randn_bf16_torch((cap, cfg.H), 24)}
    host = {k: host_bf16(v) for k, v in dev.items()}
    g_recv_w = np.random.default_rng(25).standard_normal(cap, dtype=np.float32)
    _dense_case(r.topk_idx, cfg.E, cfg.A, cfg.H, cap, host["x"], r.topk_weights,
                host["rows"], host["g_result"], host["g_recv"], g_recv_w,
                f"{name}-dense-full", dev=dev)


@pytest.mark.parametrize("name,T,H", [
    ("tiny", 256, 512), ("mixtral", 1000, 4096), ("qwen3", 777, 2048), ("dsv3", 501, 7168),
    ("dsv3", 2049, 1032),
    # routings that break the flag's statement: still exact
    ("masked", 3001, 1024), ("masked_hot", 3001, 1024),
])
def test_dense_reduced(name, T, H):
    cfg = workloads.CONFIGS[name]
    cap = oracle.recv_capacity_worst(T, cfg.K, cfg.E, cfg.A)
    c, r, x, rows, g_result, g_recv, g_recv_w = _inputs(cfg, T, H, cap, seed=3)
    _dense_case(r.topk_idx, c.E, c.A, H, cap, x, r.topk_weights, rows, g_result, g_recv,
                g_recv_w, f"{name}-dense-reduced")


@pytest.mark.parametrize("label,T,K,E,A,H,recipe", EDGE, ids=[e[0] for e in EDGE])
def test_dense_edge_cases(label, T, K, E, A, H, recipe):
    rng = np.random.default_rng(zlib.crc32(("dense" + label).encode()))
    idx = _edge_ids(rng, T, K, E, recipe)
    cap = T * K + E * (A - 1)
    x, w, rows, g_result, g_recv, g_recv_w = _random_payloads(rng, T, H, cap, K)
    _dense_case(idx, E, A, H, cap, x, w, rows, g_result, g_recv, g_recv_w, label + "-dense")


@pytest.mark.parametrize("T", [1, 5, 8, 9, 63, 2047, 2048, 2049])
def test_dense_chunk_boundaries(T):
    """Token counts around the chunk and stream boundaries (chunks of
    ceil(T/8) tokens up to 256, dealt to eight streams)."""
    rng = np.random.default_rng(T)
    K, E, A, H = 4, 24, 8, 72
    idx = _edge_ids(rng, T, K, E, "uniform")
    cap = T * K + E * (A - 1)
    x, w, rows, g_result, g_recv, g_recv_w = _random_payloads(rng, T, H, cap, K)
    _dense_case(idx, E, A, H, cap, x, w, rows, g_result, g_recv, g_recv_w, f"chunks-T{T}")


@pytest.mark.parametrize("cap_frac", [0.5, 0.0])
def test_dense_overflow(cap_frac):
    rng = np.random.default_rng(12)
    T, K, E, A, H = 600, 8, 32, 16, 64
    idx = _edge_ids(rng, T, K, E, "uniform")
    cap = int((T * K + E * (A - 1)) * cap_frac)
    x, w, rows, g_result, g_recv, g_recv_w = _random_payloads(rng, T, H, cap, K)
    p = _dense_case(idx, E, A, H, cap, x, w, rows, g_result, g_recv, g_recv_w,
                    f"dense-overflow-{cap_frac}")
    assert p.status == oracle.STATUS_OVERFLOW


@pytest.mark.parametrize("dt", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("fill_pads", [True, False])
@pytest.mark.parametrize("name,T,H", [("dsv3", 300, 1024), ("qwen3", 500, 512),
                                     ("mixtral", 400, 264)])
def test_dense_payload_types_and_pad_policy(dt, fill_pads, name, T, H):
    c = workloads.scaled(workloads.CONFIGS[name], T=T, H=H)
    r = workloads.make_routing(c)
    cap = oracle.recv_capacity_worst(T, c.K, c.E, c.A)
    run_case(name + "-dense", r.topk_idx, c.E, c.A, H, cap, dt, fill_pads,
             np.random.default_rng(zlib.crc32(f"{name}{dt}{fill_pads}dense".encode())),
             dense=True)


@pytest.mark.parametrize("fill_pads", [True, False])
@pytest.mark.parametrize("T,H", [(1, 6144), (9, 6152), (300, 6144), (2049, 6152)])
def test_dense_long_rows(T, H, fill_pads):
    """Rows of 12 KiB and more, where the copy takes three pieces per wavefront
    when it also fills the pads (four otherwise): 6144 is exactly 12 pieces,
    6152 has a ragged 13th; token counts around the chunk boundaries."""
    rng = np.random.default_rng(zlib.crc32(f"long{T}-{H}-{fill_pads}".encode()))
    K, E, A = 8, 64, 16
    idx = _edge_ids(rng, T, K, E, "uniform")
    cap = T * K + E * (A - 1)
    run_case(f"long-T{T}-H{H}", idx, E, A, H, cap, "bf16", fill_pads, rng, dense=True)
