"""Host-side logic of the benchmark: algorithmic byte counts on a tiny
hand-worked routing, and the attribution of profiled kernel dispatches to ops."""
import numpy as np
import pytest

import bench


def test_algorithmic_bytes_hand_worked():
    # T=3, K=2, E=2, H=8 (B = 16 bytes per row). Token 0 -> experts 0,1;
    # token 1 -> expert 1 and a masked route; token 2 masked entirely.
    idx = np.array([[0, 1], [1, -1], [-1, -1]], np.int64)
    counts = np.array([1, 2], np.int32)
    # alignment 4: segments of 4 rows each, so 8 rows in all, 5 of them pads
    offsets = np.array([0, 4, 8], np.int32)
    b = bench.algorithmic_bytes(3, 2, 2, 8, idx, counts, offsets)
    R, P, T_act, B = 3, 5, 2, 16
    assert (b["_R"], b["_P"], b["_T_act"], b["_total"]) == (R, P, T_act, 8)
    assert b["dispatch"] == T_act * B + 8 * B + 4 * R + 8 * 8
    assert b["combine"] == R * B + 3 * B + 4 * 6
    assert b["combine_bwd"] == T_act * B + 8 * B + 4 * 8
    assert b["dispatch_bwd"] == R * B + 4 * R + 3 * B + 8 * 6
    assert b["prepare"] == 8 * 6 + 4 * 6 + 4 * 8 + 8 * 2
    assert b["combine_weighted"] == R * B + 4 * R + 3 * B + 4 * 6
    assert b["combine_weighted_bwd"] == (T_act * B + R * B + 4 * R + 8 * B + 4 * 8 + 4 * 6
                                         + 4 * P)


def test_variant_bytes():
    idx = np.array([[0, 1], [1, -1], [-1, -1]], np.int64)
    counts = np.array([1, 2], np.int32)
    offsets = np.array([0, 4, 8], np.int32)
    R, P, T_act = 3, 5, 2
    # fp32 rows: B = 32 bytes; no pad fill: pads neither written nor mapped
    b = bench.algorithmic_bytes(3, 2, 2, 8, idx, counts, offsets, esize=4, fill_pads=False)
    assert b["dispatch"] == T_act * 32 + R * 32 + 4 * R + 8 * R
    assert b["combine_bwd"] == T_act * 32 + R * 32 + 4 * R
    assert b["combine"] == R * 32 + 3 * 32 + 4 * 6
    assert b["prepare"] == 8 * 6 + 4 * 6 + 4 * (R + P) + 8 * 2
    assert bench.base_op("dispatch_nopad") == "dispatch"
    assert bench.base_op("combine_bwd_nopad") == "combine_bwd"
    assert bench.base_op("combine_fp32") == "combine"
    assert bench.base_op("combine_weighted_bwd") == "combine_weighted_bwd"
    for op in bench.EXTRA_OPS:
        assert bench.base_op(op) in b and op in bench.KERNEL_OF_OP


def test_attribution_follows_the_launch_schedule():
    names = ["epmi::run_rows_kernel<3>", "epmi::reduce_rows_kernel<8, false, 0>",
             "epmi::run_rows_kernel<3>", "epmi::reduce_rows_kernel<8, true, 0>",
             "epmi::run_wbwd_kernel<0, true>", "epmi::run_rows_kernel<4>"]
    sched = ["dispatch", "combine", "dispatch_fp32", "combine_weighted",
             "combine_weighted_bwd", "combine_bwd_nopad"]
    assert bench.attribute(names, sched) == sched
    with pytest.raises(SystemExit):
        bench.attribute(names, sched[:-1])           # a launch missing from the record
    with pytest.raises(SystemExit):
        bench.attribute(names, ["combine"] + sched[1:])   # a copy recorded as combine


def test_attribution_of_cold_launches():
    # launches timed after a cache flush carry the op name with a suffix and
    # run the op's own kernel
    names = ["epmi::run_rows_kernel<3>", "epmi::reduce_rows_kernel<8, false, 0>"]
    sched = ["dispatch" + bench.COLD, "combine" + bench.COLD]
    assert bench.attribute(names, sched) == sched
    assert bench.kernel_of("dispatch" + bench.COLD) == "run_rows_kernel"
    assert bench.kernel_of("combine") == "reduce_rows_kernel"
