"""GPU parity of prepare across its two ways of finding each unit's start.

prepare's histogram kernel writes one row of per-expert counts per unit of
512 routes and one row of sums per block of units (4, or 8 past 256 units).
Up to 64 block rows, every block of the slot kernel sums them itself; past
that, a column scan over the block rows takes its own launch, so that the
work stays linear in the routes. Where the slot kernel's blocks hold fewer
units than the histogram kernel's, a block also adds the unit rows between
the start of its histogram block and its first unit. These cases sit on both
sides of the 64-row switch, with 100, 256 and 2048 experts, masked routes
and ragged tails, for chunks of 4, 2 and 1 units (whose run entries are
built in the slot kernel or in a launch of their own, their list starts
summed there or taken from the column scan), and on both sides of the
slot kernel's block sizing (one chunk a block, or more while the grid would
outnumber the CUs or a block has fewer threads than experts), and compare
counts, offsets, slot map, row map, run entries and status with the oracle
bit for bit; two also run dispatch and combine on the prepared handle.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
from gpu_harness import GpuRun, check_all_ops, check_prepare, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build()


def _routing(label, T, K, E, masked):
    rng = np.random.default_rng(zlib.crc32(label.encode()))
    # K distinct experts per token (argpartition of random keys)
    idx = np.argpartition(rng.random((T, E)), K - 1, axis=1)[:, :K].astype(np.int64)
    if masked:
        idx[rng.random((T, K)) < masked] = -1
    return idx


# label, T, K, E, A, masked fraction; block rows = ceil(ceil(T K / 512) / 8)
# past 256 units
CASES = [
    ("direct_64_rows", 32768, 8, 256, 128, 0.0),     # 512 units, 64 block rows
    ("scan_65_rows", 32769, 8, 256, 128, 0.0),       # 513 units, 65 rows
    ("scan_odd_experts", 40000, 7, 100, 3, 0.1),     # 547 units, 69 rows
    ("direct_wide_experts", 20000, 8, 2048, 1, 0.0),  # 313 units, 40 rows
    ("scan_wide_experts", 66000, 8, 2048, 16, 0.2),  # 1032 units, 129 rows
    ("scan_masked_1m", 131072, 8, 256, 128, 0.875),  # 2048 units, 256 rows
    # the slot kernel's blocks: one chunk each while that gives no more
    # blocks than the 256 CUs and a thread per expert, else larger
    ("slot_blocks_at_cus", 65536, 8, 128, 16, 0.0),    # 1024 units, 256 blocks of 4
    ("slot_blocks_past_cus", 65600, 8, 128, 16, 0.0),  # 1025 units, blocks of 8
    ("slot_blocks_per_expert", 4096, 8, 300, 2, 0.3),  # 64 units, 300 experts
]


# the layout's row sets the chunk size (token rows of a chunk at most
# 3.5 MiB): 128-byte rows take 4 units a chunk, fp32 rows of 28 KiB 2 and
# fp32 rows of 56 KiB 1; the run entries are built in the slot kernel where
# its LDS holds a block's chunks, else in a launch of their own
ROWS = [(64, "bf16"), (7168, "fp32"), (14336, "fp32")]


@pytest.mark.parametrize("H,dt", ROWS, ids=["row128B", "row28KiB", "row56KiB"])
@pytest.mark.parametrize("label,T,K,E,A,masked", CASES, ids=[c[0] for c in CASES])
def test_prepare_both_scan_forms(label, T, K, E, A, masked, H, dt):
    idx = _routing(label, T, K, E, masked)
    cap = oracle.recv_capacity_worst(T, K, E, A)
    log(f"prepare {label}: T={T} K={K} E={E} A={A} cap={cap} units={-(-T * K // 512)} "
        f"row {H} {dt}")
    run = GpuRun(idx, E, A, H, cap, prepare_dtype=dt)
    run.prepare()
    p = oracle.prepare(idx, E, A, cap)
    check_prepare(run, p)
    # a second prepare on the same handle (scratch rows of the first left in
    # place) gives the same maps
    run.prepare()
    check_prepare(run, p)


@pytest.mark.parametrize("label", ["scan_65_rows", "scan_wide_experts"])
def test_payload_ops_after_scanned_prepare(label):
    _, T, K, E, A, masked = next(c for c in CASES if c[0] == label)
    H = 136
    idx = _routing(label, T, K, E, masked)
    cap = oracle.recv_capacity_worst(T, K, E, A)
    rng = np.random.default_rng(7)
    x = rng.integers(0, 1 << 16, size=(T, H), dtype=np.uint16)
    x[(x & 0x7F80) == 0x7F80] = 0x3F80            # no NaN or Inf payloads
    w = rng.standard_normal((T, K)).astype(np.float32)
    rows = rng.integers(0, 1 << 16, size=(cap, H), dtype=np.uint16)
    rows[(rows & 0x7F80) == 0x7F80] = 0x3F80
    g_result = rng.integers(0, 1 << 16, size=(T, H), dtype=np.uint16)
    g_result[(g_result & 0x7F80) == 0x7F80] = 0x3F80
    g_recv = rows[::-1].copy()
    g_recv_w = rng.standard_normal(cap).astype(np.float32)
    run = GpuRun(idx, E, A, H, cap)
    run.prepare()
    p = oracle.prepare(idx, E, A, cap)
    check_prepare(run, p)
    check_all_ops(run, p, x, w, rows, g_result, g_recv, g_recv_w, label=label)
