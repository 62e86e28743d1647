#!/usr/bin/env python3
"""Benchmark of the expert-parallel routing hot path on one MI355X.

One step = one pass of the whole path over one batch: prepare, dispatch,
combine, combine_bwd and dispatch_bwd on the DeepSeek-V3-shaped workload
(T=4096 tokens, H=7168 bf16, E=256 experts, top-8 group-limited routing,
alignment 128), with every input resident in HBM before timing starts.

The headline is dispatch+combine throughput in algorithmic HBM GB/s (bytes
the method must move, see ``algorithmic_bytes``) over their kernel time,
measured with HIP events recorded on the stream the kernels run on. The line
also carries the roofline of the dominant kernel and the CPU oracle timed on a
bounded sample of the same workload on this host.

After the step, the variants outside it are timed the same way, one op at a
time, and reported under "ops_outside_step": the fused weighted combine and
its backward, dispatch and combine_bwd without the pad fill, combine on fp16
payloads, dispatch and combine on fp32 payloads.

Then the memory-pattern ceilings of the same device (``--no-ceilings`` skips
them) are timed from ``libep_ceilings.so``, kernels that move bytes in the
routing ops' access patterns with no routing at all: a dense write front, rows
of the workload's size written in a scrambled order (dispatch's write
pattern), a dense read front, a dense copy, and K hashed rows summed per token
(combine's pattern at full density). They are reported under "ceilings" with
each headline op's bandwidth as a fraction of its pattern's ceiling.

    python bench.py [--steps K] [--warmup W] [--workload dsv3] [--no-cpu-baseline]

Profiling (rocprofv3 on an MI355X, then summarised here):
    --schedule-out FILE   record, in launch order, the op of every payload
                          kernel launch (prepare excluded), so that profiled
                          dispatches can be attributed to ops
    --summarize-trace DIR / --summarize-pmc FETCH_DIR WRITE_DIR
                          write the profiles/ summaries from rocprofv3 output
                          directories that hold such a schedule.json
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = [os.path.join(ROOT, "combine_ep_prepare_amd", "csrc", f)
                  for f in ("ep_kernels.hip", "ep_api.hip", "ep_internal.h")]

STEP_OPS = ["prepare", "dispatch", "combine", "combine_bwd", "dispatch_bwd"]
CEILINGS_LIB = os.path.join(ROOT, "combine_ep_prepare_amd", "libep_ceilings.so")
CEILING_BUFFER_BYTES = 1 << 30     # each pattern moves 1 GiB (or the largest fit)

# op -> the library kernel that runs it
KERNEL_OF_OP = {"dispatch": "run_rows_kernel", "combine_bwd": "run_rows_kernel",
                "combine": "reduce_rows_kernel", "dispatch_bwd": "reduce_rows_kernel",
                "combine_weighted": "reduce_rows_kernel",
                "combine_weighted_bwd": "run_wbwd_kernel",
                "dispatch_nopad": "run_rows_kernel",
                "combine_bwd_nopad": "run_rows_kernel",
                "combine_fp16": "reduce_rows_kernel",
                "dispatch_fp32": "run_rows_kernel",
                "combine_fp32": "reduce_rows_kernel"}
PAYLOAD_KERNELS = ("scatter_rows_kernel", "reduce_rows_kernel", "weighted_bwd_kernel",
                   "run_rows_kernel", "run_wbwd_kernel")
PREPARE_KERNELS = ("prepare_hist_kernel", "prepare_slots_kernel", "prepare_fused_kernel",
                   "prepare_runs_kernel")

COLD = "@cold"      # suffix of the launches timed after a cache flush


def kernel_of(op: str) -> str:
    """The library kernel that runs ``op`` (a cold launch runs the op's
    kernel)."""
    op = op[:-len(COLD)] if op.endswith(COLD) else op
    return KERNEL_OF_OP[op]

# ops timed after the step: op -> (payload type, pads filled); the fp32 ops
# use a handle prepared with the fp32 layout (its run chunks sized for fp32
# rows), as a caller with fp32 payloads would prepare it
EXTRA_OPS = {"combine_weighted": ("bf16", True),
             "combine_weighted_bwd": ("bf16", True),
             "dispatch_nopad": ("bf16", False), "combine_bwd_nopad": ("bf16", False),
             "combine_fp16": ("fp16", True), "dispatch_fp32": ("fp32", True),
             "combine_fp32": ("fp32", True)}
ESIZE = {"bf16": 2, "fp16": 2, "fp32": 4}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """C/C++ source without comments, trailing blanks and empty lines."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip())


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code (comments ignored): profiles taken on
    other code are not used."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p) as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def algorithmic_bytes(T, K, E, H, topk_idx, counts_np, offsets_np, esize=2, fill_pads=True):
    """Bytes each op must move at minimum (each row once).

    B = esize*H bytes per row, R valid routes, P pad rows (Pw = P when pads
    are filled, else 0), T_act tokens with at least one valid route.
      dispatch      T_act*B + (R+Pw)*B + 4R + 8(R+Pw)  rows, weights in/out, row map
      combine       R*B + T*B + 4TK                    rows in/out, slot map
      combine_bwd   T_act*B + (R+Pw)*B + 4(R+Pw)       rows in/out, row map
      dispatch_bwd  R*B + 4R + T*B + 8TK               rows in/out, weights, slot map
      prepare       8TK + 4TK + 4(R+P) + 8E            ids, slots, row map, counts
      combine_weighted      R*B + 4R + T*B + 4TK       rows and weights in, rows out,
                                                       slot map
      combine_weighted_bwd  T_act*B + R*B + 4R + (R+Pw)*B + 4(R+Pw) + 4TK + 4Pw
                            grads in, expert rows and weights in, row and weight
                            grads out, slot map, pad-row list
    """
    B = esize * H
    R = int(counts_np.sum())
    total = int(offsets_np[-1])
    P = total - R
    Pw = P if fill_pads else 0
    T_act = int((topk_idx >= 0).any(axis=1).sum()) if T else 0
    return {
        "dispatch": T_act * B + (R + Pw) * B + 4 * R + 8 * (R + Pw),
        "combine": R * B + T * B + 4 * T * K,
        "combine_bwd": T_act * B + (R + Pw) * B + 4 * (R + Pw),
        "dispatch_bwd": R * B + 4 * R + T * B + 8 * T * K,
        "prepare": 8 * T * K + 4 * T * K + 4 * (R + P) + 8 * E,
        "combine_weighted": R * B + 4 * R + T * B + 4 * T * K,
        "combine_weighted_bwd": (T_act * B + R * B + 4 * R + (R + Pw) * B + 4 * (R + Pw)
                                 + 4 * T * K + 4 * Pw),
        "_R": R, "_P": P, "_T_act": T_act, "_total": total,
    }


def base_op(op: str) -> str:
    """dispatch_fp32 -> dispatch, combine_bwd_nopad -> combine_bwd, ..."""
    for suffix in ("_nopad", "_fp16", "_fp32"):
        if op.endswith(suffix):
            return op[:-len(suffix)]
    return op


def attribute(kernel_names, schedule):
    """Pair the library's payload-kernel dispatches (demangled names in
    dispatch order, all other kernels already left out) with the ops recorded
    in launch order. Raises if the two do not line up."""
    if len(kernel_names) != len(schedule):
        raise SystemExit(f"{len(kernel_names)} payload dispatches profiled but "
                         f"{len(schedule)} launches recorded")
    for i, (name, op) in enumerate(zip(kernel_names, schedule)):
        if kernel_of(op) not in name:
            raise SystemExit(f"dispatch {i}: {name} does not run {op}")
    return list(schedule)


def _read_csv_rows(directory: str, suffix: str):
    import csv
    import glob
    rows = []
    for path in sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True)):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def _schedule(directory: str):
    """The ops of the payload launches, in launch order."""
    with open(os.path.join(directory, "schedule.json")) as f:
        d = json.load(f)
    return d["ops"]


def _recorded_cmd(directory: str) -> str:
    """The bench command line that wrote this profile directory's schedule,
    with the directory written as <dir>."""
    with open(os.path.join(directory, "schedule.json")) as f:
        argv = json.load(f).get("argv", [])
    # the path given to --schedule-out names the profile directory
    return "python3 bench.py " + " ".join(
        "<dir>/schedule.json" if a.endswith("schedule.json") else a for a in argv)


def _is_payload(name: str) -> bool:
    return any(k in name for k in PAYLOAD_KERNELS)


def _pmc_path(op: str, workload: str) -> str:
    return os.path.join(PROFILE_DIR, f"{kernel_of(op)}_{op}_{workload}_pmc.txt")


def load_traffic(op: str, workload: str, src_hash: str):
    """Measured HBM bytes per launch from a committed rocprofv3 counter summary,
    used only when it was taken on the current kernel sources."""
    path = _pmc_path(op, workload)
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            line = [ln for ln in f if ln.startswith("JSON: ")][-1]
        d = json.loads(line[len("JSON: "):])
    except (OSError, ValueError, IndexError):
        return None
    if d.get("kernel_source_hash") != src_hash:
        return None
    return d.get("hbm_bytes_per_launch")


def summarize_pmc(fetch_dir: str, write_dir: str, workload: str, copy_mib: int,
                  out_dir: str = PROFILE_DIR):
    """Turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then
    WRITE_SIZE, both with --calibration-copy-mib and --schedule-out
    <dir>/schedule.json) into per-op HBM bytes.

    Each counter is scaled by what it reads for the plain copy of known size
    (the runtime's copyBuffer kernel, which PyTorch's device-to-device copy
    uses), so the result is in true bytes. Payload dispatches are attributed
    to ops through the recorded launch schedule."""
    import numpy as np
    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _read_csv_rows(d, "counter_collection.csv")
                if r.get("Counter_Name") == counter]
        rows.sort(key=lambda r: int(r.get("Dispatch_Id", 0)))
        calib = [r for r in rows if "copybuffer" in r["Kernel_Name"].lower()
                 and float(r["Counter_Value"]) > copy_mib * 1024.0 / 8]
        if not calib:
            raise SystemExit(f"no calibration copy found for {counter} in {d}")
        expected_kib = copy_mib * 1024.0
        factor = float(np.median([float(r["Counter_Value"]) for r in calib])) / expected_kib
        pay = [r for r in rows if _is_payload(r["Kernel_Name"])]
        sched = _schedule(d)
        ops = attribute([r["Kernel_Name"] for r in pay], sched)
        per_op = {}
        for r, op in zip(pay, ops):
            per_op.setdefault(op, []).append(float(r["Counter_Value"]) / factor * 1024.0)
        res[counter] = {"factor": factor,
                        "per_op_bytes": {op: float(np.median(v)) for op, v in per_op.items()}}
    out = {"workload": workload, "kernel_source_hash": kernel_source_hash(),
           "calibration": {"copy_mib": copy_mib,
                           "fetch_factor": res["FETCH_SIZE"]["factor"],
                           "write_factor": res["WRITE_SIZE"]["factor"]}}
    cmd = ("cd /tmp && export TMPDIR=/tmp && timeout -s KILL 150 rocprofv3 --pmc <COUNTER> "
           f"-d <dir> -o pmc --output-format csv -- {_recorded_cmd(fetch_dir)}   (once with "
           "FETCH_SIZE, once with WRITE_SIZE); then python bench.py --summarize-pmc "
           f"<fetch dir> <write dir> --workload {workload} --calibration-copy-mib {copy_mib}")
    for op in KERNEL_OF_OP:                    # warm launches only
        fb = res["FETCH_SIZE"]["per_op_bytes"].get(op)
        wb = res["WRITE_SIZE"]["per_op_bytes"].get(op)
        if fb is None or wb is None:
            continue
        summary = dict(out)
        kern = kernel_of(op)
        summary.update({"op": op, "kernel": kern,
                        "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
                        "hbm_bytes_per_launch": fb + wb})
        fc = res["FETCH_SIZE"]["per_op_bytes"].get(op + COLD)
        wc = res["WRITE_SIZE"]["per_op_bytes"].get(op + COLD)
        if fc is not None and wc is not None:
            # the same op launched right after the cache flush
            summary.update({"cold_fetch_bytes_per_launch": fc, "cold_write_bytes_per_launch": wc})
        path = _pmc_path(op, workload)
        with open(path, "w") as f:
            f.write(f"# HBM traffic of {kern} ({op}), workload {workload}\n")
            f.write(f"# command: {cmd}\n")
            f.write(f"# FETCH_SIZE scale {out['calibration']['fetch_factor']:.4f}, WRITE_SIZE "
                    f"scale {out['calibration']['write_factor']:.4f} (counter / true bytes of "
                    f"a {copy_mib} MiB device copy in the same run)\n")
            f.write(f"# per launch (median over the profiled launches): fetch "
                    f"{fb / 1e6:.1f} MB, write {wb / 1e6:.1f} MB, total {(fb + wb) / 1e6:.1f} MB\n")
            f.write("JSON: " + json.dumps(summary) + "\n")
        print(f"{path}: fetch {fb / 1e6:.1f} MB write {wb / 1e6:.1f} MB", flush=True)


def summarize_trace(trace_dir: str, workload: str, steps: int, warmup: int,
                    out_dir: str = PROFILE_DIR):
    """profiles/ep_kernels_<workload>_kernel_stats.txt from a rocprofv3
    --kernel-trace --stats run of this script with --schedule-out
    <dir>/schedule.json: rocprofv3's per-kernel statistics, then the same
    dispatches grouped by op."""
    import numpy as np
    rows = _read_csv_rows(trace_dir, "kernel_stats.csv")
    trace = _read_csv_rows(trace_dir, "kernel_trace.csv")
    trace.sort(key=lambda r: int(r["Dispatch_Id"]))
    pay = [r for r in trace if _is_payload(r["Kernel_Name"])]
    sched = _schedule(trace_dir)
    ops = attribute([r["Kernel_Name"] for r in pay], sched)
    per_op = {}
    for r, op in zip(pay, ops):
        per_op.setdefault(op, []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    prep = {}
    for r in trace:
        for k in PREPARE_KERNELS:
            if k in r["Kernel_Name"]:
                prep.setdefault(k, []).append(
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    path = os.path.join(out_dir, f"ep_kernels_{workload}_kernel_stats.txt")
    cmd = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -d <dir> -o "
           f"trace --output-format csv -- {_recorded_cmd(trace_dir)}; then python bench.py "
           f"--summarize-trace <dir> --workload {workload} --steps {steps} --warmup {warmup}")
    with open(path, "w") as f:
        f.write(f"# rocprofv3 kernel statistics, workload {workload}\n")
        f.write(f"# command: {cmd}\n")
        f.write(f"# kernel source hash {kernel_source_hash()}\n")
        f.write(f"{'kernel':60s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} "
                f"{'share%':>7s}\n")
        for r in rows:
            name = r["Name"]
            short = name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
            f.write(f"{short[:60]:60s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} "
                    f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} "
                    f"{float(r['Percentage']):7.2f}\n")
        f.write("\n# the payload dispatches by op (kernel trace, launch schedule)\n")
        f.write(f"{'op':24s} {'kernel':22s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} "
                f"{'max_us':>9s}\n")
        for op, v in list(per_op.items()) + list(prep.items()):
            kern = kernel_of(op) if op.replace(COLD, "") in KERNEL_OF_OP else op
            f.write(f"{op:24s} {kern:22s} {len(v):6d} {np.mean(v):9.2f} {np.min(v):9.2f} "
                    f"{np.max(v):9.2f}\n")
    print(path, flush=True)


def cpu_baseline(cfg, r, host, cap, budget_s=12.0, threads=1):
    """The oracle as it stands on the same inputs, its row and token loops on
    ``threads`` threads (0: the OpenMP default, every core it is given):
    whole steps repeated until the time budget is spent (at least one).
    Returns (dispatch s, combine s, steps, seconds spent, threads used)."""
    import oracle
    used = oracle.set_threads(threads)
    t_d = t_c = 0.0
    n = 0
    start = time.perf_counter()
    while True:
        p = oracle.prepare(r.topk_idx, cfg.E, cfg.A, cap)
        t1 = time.perf_counter()
        oracle.dispatch(p, host["x"], r.topk_weights)
        t2 = time.perf_counter()
        oracle.combine(p, host["expert_out"])
        t3 = time.perf_counter()
        oracle.combine_bwd(p, host["g_result"])
        oracle.dispatch_bwd(p, host["g_recv"], host["g_recv_w"])
        t_d += t2 - t1
        t_c += t3 - t2
        n += 1
        if time.perf_counter() - start > budget_s:
            break
    return t_d / n, t_c / n, n, time.perf_counter() - start, used


def _ceilings_lib():
    import ctypes as C
    if not os.path.exists(CEILINGS_LIB):
        raise ImportError(f"{CEILINGS_LIB} is missing: build it with "
                          "`python -c 'import __graft_entry__ as g; g.build()'`")
    lib = C.CDLL(CEILINGS_LIB)
    i64, vp = C.c_int64, C.c_void_p
    lib.epc_write_linear.argtypes = [vp, i64, vp]
    lib.epc_write_rows.argtypes = [vp, i64, i64, vp]
    lib.epc_read_linear.argtypes = [vp, i64, vp, vp]
    lib.epc_copy_linear.argtypes = [vp, vp, i64, vp]
    lib.epc_gather_sum.argtypes = [vp, i64, i64, i64, C.c_int, vp, vp]
    lib.epc_flush.argtypes = [vp, vp, i64, vp, vp]
    for name in ("epc_write_linear", "epc_write_rows", "epc_read_linear", "epc_copy_linear",
                 "epc_gather_sum", "epc_flush"):
        getattr(lib, name).restype = C.c_int
    return lib


def ceiling_sizes(T, K, H, esize=2, budget=CEILING_BUFFER_BYTES):
    """Sizes of the ceiling patterns for a workload: rows of the workload's
    payload row, as many as fit the budget (a power of two for the scrambled
    write), and the dense gather of T tokens x K rows when K is 1, 2, 4 or 8
    and the rows fit."""
    row = H * esize
    nrows = 1
    while nrows * 2 * row <= budget:
        nrows *= 2
    gather = None
    if K in (1, 2, 4, 8) and T * K * row <= budget:
        gather = {"ntok": T, "k": K, "nrows": T * K, "row_bytes": row,
                  "bytes": T * K * row + T * row}
    return {"row_bytes": row, "write_rows": nrows, "write_rows_bytes": nrows * row,
            "gather": gather}


def measure_ceilings(T, K, H, launches, warmup):
    """GB/s of each memory pattern on the current device and stream."""
    import torch
    lib = _ceilings_lib()
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    nb = CEILING_BUFFER_BYTES
    a = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    b = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    sz = ceiling_sizes(T, K, H)

    def timed(fn, nbytes):
        for _ in range(warmup):
            assert fn() == 0
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(launches):
            assert fn() == 0
        e1.record(stream)
        torch.cuda.synchronize()
        return round(nbytes / (e0.elapsed_time(e1) * 1e-3 / launches) / 1e9, 1)

    out = {"unit": "GB/s", "row_bytes": sz["row_bytes"], "launches": launches}
    out["linear_write"] = timed(lambda: lib.epc_write_linear(a.data_ptr(), nb, sp), nb)
    out["scattered_row_write"] = timed(
        lambda: lib.epc_write_rows(a.data_ptr(), sz["write_rows"], sz["row_bytes"], sp),
        sz["write_rows_bytes"])
    out["linear_read"] = timed(lambda: lib.epc_read_linear(a.data_ptr(), nb, sink.data_ptr(), sp),
                               nb)
    out["linear_copy"] = timed(lambda: lib.epc_copy_linear(a.data_ptr(), b.data_ptr(), nb, sp),
                               2 * nb)
    g = sz["gather"]
    if g is not None:
        out["gather_sum"] = timed(
            lambda: lib.epc_gather_sum(a.data_ptr(), g["nrows"], g["row_bytes"], g["ntok"],
                                       g["k"], b.data_ptr(), sp), g["bytes"])
    del a, b, sink
    torch.cuda.synchronize()
    return out


PREPARE_SWEEP_T = (256, 512, 1024, 2048, 4096, 16384, 65536, 131072, 262144, 524288)


def prepare_sweep(workload: str, steps: int, warmup: int):
    """prepare's time against the number of routes: the workload's routing
    recipe at several token counts, prepare timed alone (back to back, HIP
    events on its stream), one JSON line."""
    import numpy as np
    import torch

    import combine_ep_prepare_amd as ep
    import workloads

    torch.cuda.set_device(0)
    base = workloads.CONFIGS[workload]
    stream = torch.cuda.current_stream()
    points = []
    for T in PREPARE_SWEEP_T:
        cfg = workloads.scaled(base, T=T)
        r = workloads.make_routing(cfg)
        cap = ep.recv_capacity_worst(T, cfg.K, cfg.E, cfg.A)
        L = ep.Layout(T, cfg.K, cfg.E, cfg.A, cfg.H, cap)
        handle = ep.new_handle(L)
        idx = torch.from_numpy(r.topk_idx).cuda()
        counts = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
        offsets = torch.empty(cfg.E + 1, dtype=torch.int32, device="cuda")
        for _ in range(warmup):
            ep.prepare(L, idx, counts, handle, offsets)
        evs = []
        for _ in range(steps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            ep.prepare(L, idx, counts, handle, offsets)
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        assert ep.read_status(handle) & ~ep.STATUS_OVERFLOW == 0
        us = [a.elapsed_time(b) * 1e3 for a, b in evs]
        routes = T * cfg.K
        points.append({"T": T, "routes": routes, "units": -(-routes // 512),
                       "avg_us": round(float(np.mean(us)), 2),
                       "median_us": round(float(np.median(us)), 2),
                       "ns_per_route": round(float(np.median(us)) * 1e3 / routes, 3)})
        log(f"prepare T={T}: {points[-1]['median_us']} us")
        del handle, idx
    print(json.dumps({"metric": "prepare_us_vs_routes", "workload": workload, "K": base.K,
                      "E": base.E, "A": base.A, "steps": steps, "warmup": warmup,
                      "points": points}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra-ops", action="store_true",
                    help="skip timing the ops outside the step")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip timing the memory-pattern ceilings")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of CPU oracle work per thread setting (all cores, one)")
    ap.add_argument("--cold-steps", type=int, default=None,
                    help="steps timed with the caches flushed before every op "
                         "(default: --steps; 0 skips them)")
    ap.add_argument("--flush-mib", type=int, default=512,
                    help="MiB written, then MiB of another buffer read, before each cold op")
    ap.add_argument("--headline", choices=("warm", "cold"), default="warm",
                    help="which timing protocol `value` reports")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="run a plain device copy of this size first (counter calibration)")
    ap.add_argument("--schedule-out", metavar="FILE",
                    help="write the op of every payload kernel launch, in order, as JSON")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured in one HIP graph and replayed")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/*_pmc.txt from two rocprofv3 counter runs")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="write profiles/*_kernel_stats.txt from a rocprofv3 --stats run")
    ap.add_argument("--prepare-sweep", action="store_true",
                    help="time prepare alone on the workload's routing recipe at token "
                         "counts from 256 to 524288 and print one JSON line")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload,
                      args.calibration_copy_mib)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.workload, args.steps, args.warmup)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU's share of the path; the library has no "
              "multi-GPU path, so only --gpus 1 runs.", file=sys.stderr)
        sys.exit(2)
    if args.prepare_sweep:
        prepare_sweep(args.workload, args.steps, args.warmup)
        return

    import numpy as np
    import torch

    import combine_ep_prepare_amd as ep
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    cfg = workloads.CONFIGS[args.workload]
    T, K, E, A, H = cfg.T, cfg.K, cfg.E, cfg.A, cfg.H
    log(f"workload {cfg.name}: T={T} H={H} E={E} K={K} A={A}")
    r = workloads.make_routing(cfg)
    cap = ep.recv_capacity_worst(T, K, E, A)
    dense = bool((r.topk_idx >= 0).all())       # reported only
    L = ep.Layout(T, K, E, A, H, cap)
    dev = torch.device("cuda")
    handle = ep.new_handle(L)
    idx = torch.from_numpy(r.topk_idx).to(dev)
    w = torch.from_numpy(r.topk_weights).to(dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    x = workloads.randn_bf16_torch((T, H), 1)
    recv = torch.zeros(cap, H, dtype=torch.bfloat16, device=dev)
    recv_w = torch.zeros(cap, dtype=torch.float32, device=dev)
    result = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    g_result = workloads.randn_bf16_torch((T, H), 2)
    g_exp = torch.empty(cap, H, dtype=torch.bfloat16, device=dev)
    g_recv = workloads.randn_bf16_torch((cap, H), 3)
    g_recv_w = workloads.randn_bf16_torch((cap,), 4).float()
    g_tok = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    g_w = torch.empty(T, K, dtype=torch.float32, device=dev)
    schedule = []          # op of every payload kernel launch, in order

    # The experts' stand-in: expert_out = bf16(recv * recv_topk_weights),
    # computed once outside the timed region (the caller's pre-multiply).
    ep.prepare(L, idx, counts, handle, offsets)
    schedule.append("dispatch")
    ep.dispatch(L, handle, x, w, recv, recv_w)
    expert_out = (recv.float() * recv_w[:, None]).to(torch.bfloat16)
    torch.cuda.synchronize()
    counts_np = counts.cpu().numpy()
    offsets_np = offsets.cpu().numpy()
    nbytes = algorithmic_bytes(T, K, E, H, r.topk_idx, counts_np, offsets_np)
    log(f"R={nbytes['_R']} P={nbytes['_P']} total={nbytes['_total']} cap={cap} "
        f"T_act={nbytes['_T_act']}")

    if args.calibration_copy_mib:
        n = args.calibration_copy_mib << 19          # bf16 elements
        src_c = torch.empty(n, dtype=torch.bfloat16, device=dev).normal_()
        dst_c = torch.empty_like(src_c)
        for _ in range(3):
            dst_c.copy_(src_c)
        torch.cuda.synchronize()
        del src_c, dst_c

    stream = torch.cuda.current_stream()
    step_fns = [
        ("prepare", lambda: ep.prepare(L, idx, counts, handle, offsets)),
        ("dispatch", lambda: ep.dispatch(L, handle, x, w, recv, recv_w)),
        ("combine", lambda: ep.combine(L, handle, expert_out, result)),
        ("combine_bwd", lambda: ep.combine_bwd(L, handle, g_result, g_exp)),
        ("dispatch_bwd", lambda: ep.dispatch_bwd(L, handle, g_recv, g_recv_w, g_tok, g_w)),
    ]

    def step(ev=None):
        for j, (op, fn) in enumerate(step_fns):
            if ev is not None:
                ev[j].record(stream)
            if op != "prepare":
                schedule.append(op)
            fn()
        if ev is not None:
            ev[len(step_fns)].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert ep.read_status(handle) == 0, "unexpected status bits"

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(step_fns) + 1)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    per_op_ms = {op: [] for op in STEP_OPS}
    for ev in events:
        for j, op in enumerate(STEP_OPS):
            per_op_ms[op].append(ev[j].elapsed_time(ev[j + 1]))
    avg = {op: float(np.mean(v)) for op, v in per_op_ms.items()}
    med = {op: float(np.median(v)) for op, v in per_op_ms.items()}
    p10 = {op: float(np.percentile(v, 10)) for op, v in per_op_ms.items()}
    p90 = {op: float(np.percentile(v, 90)) for op, v in per_op_ms.items()}

    # Cold: the same five ops, each preceded on the same stream (no host gap)
    # by a flush that writes one buffer and then reads another, each larger
    # than the 256 MB Infinity Cache, with plain cache-allocating accesses. The
    # op then finds none of its inputs in the L2s or the Infinity Cache, and
    # no dirty line of the op before it is left to write back meanwhile.
    cold_steps = args.steps if args.cold_steps is None else args.cold_steps
    cold_avg = cold_med = None
    if cold_steps > 0:
        clib = _ceilings_lib()
        fbytes = args.flush_mib << 20
        fl_a = torch.empty(fbytes, dtype=torch.uint8, device=dev)
        fl_b = torch.zeros(fbytes, dtype=torch.uint8, device=dev)
        fl_sink = torch.zeros(1024, dtype=torch.uint8, device=dev)
        sp = stream.cuda_stream

        def flush():
            assert clib.epc_flush(fl_a.data_ptr(), fl_b.data_ptr(), fbytes,
                                  fl_sink.data_ptr(), sp) == 0

        cev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in step_fns] for _ in range(cold_steps)]
        torch.cuda.synchronize()
        for i in range(cold_steps):
            for j, (op, fn) in enumerate(step_fns):
                flush()
                cev[i][j][0].record(stream)
                if op != "prepare":
                    schedule.append(op + COLD)
                fn()
                cev[i][j][1].record(stream)
        torch.cuda.synchronize()
        assert ep.read_status(handle) == 0, "unexpected status bits"
        cold_ms = {op: [cev[i][j][0].elapsed_time(cev[i][j][1]) for i in range(cold_steps)]
                   for j, (op, _) in enumerate(step_fns)}
        cold_avg = {op: float(np.mean(v)) for op, v in cold_ms.items()}
        cold_med = {op: float(np.median(v)) for op, v in cold_ms.items()}
        del fl_a, fl_b, fl_sink

    # The same step captured once in a HIP graph and replayed: the GPU time of
    # the five ops without the host's launch gaps (what a small, launch-bound
    # routing costs inside a captured layer). Not under the profiler's launch
    # schedule: replays are not recorded in it.
    graph = None
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for _ in range(2):
                for _, fn in step_fns:
                    fn()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _, fn in step_fns:
                fn()
        for _ in range(args.warmup):
            g.replay()
        gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        for a, b in gev:
            a.record(stream)
            g.replay()
            b.record(stream)
        torch.cuda.synchronize()
        gv = [a.elapsed_time(b) for a, b in gev]
        assert ep.read_status(handle) == 0, "unexpected status bits"
        graph = {"step_us_median": round(float(np.median(gv)) * 1e3, 2),
                 "step_us_avg": round(float(np.mean(gv)) * 1e3, 2),
                 "eager_step_us_avg": round(sum(avg[op] for op in STEP_OPS) * 1e3, 2),
                 "replays": args.steps}
        del g

    # Ops outside the step, timed one at a time over the same number of
    # launches after the same warmup.
    extra = {}
    if not args.no_extra_ops:
        lay = {key: ep.Layout(T, K, E, A, H, cap, dtype=key[0], fill_pads=key[1])
               for key in set(EXTRA_OPS.values())}
        # the fp32 ops' own handle, prepared with the fp32 layout
        handle32 = ep.new_handle(lay[("fp32", True)])
        counts32 = torch.empty(E, dtype=torch.int32, device=dev)
        ep.prepare(lay[("fp32", True)], idx, counts32, handle32)
        result_w = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
        g_rows_w = torch.empty(cap, H, dtype=torch.bfloat16, device=dev)
        g_recv_w2 = torch.empty(cap, dtype=torch.float32, device=dev)
        recv_np = torch.empty(cap, H, dtype=torch.bfloat16, device=dev)
        recv_w_np = torch.empty(cap, dtype=torch.float32, device=dev)
        g_exp_np = torch.empty(cap, H, dtype=torch.bfloat16, device=dev)
        eo16 = expert_out.to(torch.float16)
        res16 = torch.empty(T, H, dtype=torch.float16, device=dev)
        x32 = x.float()
        recv32 = torch.empty(cap, H, dtype=torch.float32, device=dev)
        recv_w32 = torch.empty(cap, dtype=torch.float32, device=dev)
        eo32 = expert_out.float()
        res32 = torch.empty(T, H, dtype=torch.float32, device=dev)
        fns = {
            "combine_weighted": lambda Lx: ep.combine_weighted(Lx, handle, recv, recv_w,
                                                               result_w),
            "combine_weighted_bwd": lambda Lx: ep.combine_weighted_bwd(
                Lx, handle, g_result, recv, recv_w, g_rows_w, g_recv_w2),
            "dispatch_nopad": lambda Lx: ep.dispatch(Lx, handle, x, w, recv_np, recv_w_np),
            "combine_bwd_nopad": lambda Lx: ep.combine_bwd(Lx, handle, g_result, g_exp_np),
            "combine_fp16": lambda Lx: ep.combine(Lx, handle, eo16, res16),
            "dispatch_fp32": lambda Lx: ep.dispatch(Lx, handle32, x32, w, recv32, recv_w32),
            "combine_fp32": lambda Lx: ep.combine(Lx, handle32, eo32, res32),
        }
        for op, key in EXTRA_OPS.items():
            dt, fill = key[0], key[1]
            Lx = lay[key]
            fn = fns[op]
            for _ in range(args.warmup):
                schedule.append(op)
                fn(Lx)
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.steps)]
            torch.cuda.synchronize()
            for a, b in evs:
                a.record(stream)
                schedule.append(op)
                fn(Lx)
                b.record(stream)
            torch.cuda.synchronize()
            v = [a.elapsed_time(b) for a, b in evs]
            avg[op] = float(np.mean(v))
            med[op] = float(np.median(v))
            p10[op] = float(np.percentile(v, 10))
            p90[op] = float(np.percentile(v, 90))
            nb = algorithmic_bytes(T, K, E, H, r.topk_idx, counts_np, offsets_np,
                                   esize=ESIZE[dt], fill_pads=fill)
            extra[op] = nb[base_op(op)]
        assert ep.read_status(handle) == 0, "unexpected status bits"

    if args.schedule_out:
        os.makedirs(os.path.dirname(os.path.abspath(args.schedule_out)), exist_ok=True)
        with open(args.schedule_out, "w") as f:
            json.dump({"ops": schedule, "argv": sys.argv[1:]}, f)

    def gbs(op, nb):
        return nb / (avg[op] * 1e-3) / 1e9

    pair_bytes = nbytes["dispatch"] + nbytes["combine"]
    warm_pair_s = (avg["dispatch"] + avg["combine"]) * 1e-3
    warm = {"pair_GBps": round(pair_bytes / warm_pair_s / 1e9, 1),
            "pct_of_peak": round(100 * pair_bytes / warm_pair_s / 1e9 / HBM_PEAK_GBS, 2),
            "dispatch_us": round(avg["dispatch"] * 1e3, 2),
            "combine_us": round(avg["combine"] * 1e3, 2),
            "protocol": "ops back to back inside whole steps"}
    cold = None
    if cold_avg is not None:
        cold_pair_s = (cold_avg["dispatch"] + cold_avg["combine"]) * 1e-3
        cold = {"pair_GBps": round(pair_bytes / cold_pair_s / 1e9, 1),
                "pct_of_peak": round(100 * pair_bytes / cold_pair_s / 1e9 / HBM_PEAK_GBS, 2),
                "dispatch_us": round(cold_avg["dispatch"] * 1e3, 2),
                "combine_us": round(cold_avg["combine"] * 1e3, 2),
                "protocol": f"each op after a flush ({args.flush_mib} MiB written, then "
                            f"{args.flush_mib} MiB of another buffer read, same stream)",
                "steps": cold_steps,
                "ops": {op: {"avg_us": round(cold_avg[op] * 1e3, 2),
                             "median_us": round(cold_med[op] * 1e3, 2),
                             "GBps": (round(nbytes[op] / (cold_avg[op] * 1e-3) / 1e9, 1)
                                      if op != "prepare" else None)}
                        for op in STEP_OPS}}
    if args.headline == "cold" and cold is None:
        raise SystemExit("--headline cold needs --cold-steps > 0")
    pair_s = cold_pair_s if args.headline == "cold" else warm_pair_s
    value = pair_bytes / pair_s / 1e9
    dominant = max(("dispatch", "combine", "combine_bwd", "dispatch_bwd"),
                   key=lambda op: avg[op])
    src_hash = kernel_source_hash()
    traffic = load_traffic(dominant, cfg.name, src_hash)
    achieved = gbs(dominant, nbytes[dominant])
    roofline = {"bound": "hbm", "kernel": f"{kernel_of(dominant)} ({dominant})",
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic,
                "algorithmic_bytes_per_launch": nbytes[dominant],
                "avg_launch_us": round(avg[dominant] * 1e3, 2)}

    ceilings = None
    if not args.no_ceilings:
        ceilings = measure_ceilings(T, K, H, args.steps, args.warmup)
        ceilings["dispatch_frac_of_scattered_row_write"] = round(
            gbs("dispatch", nbytes["dispatch"]) / ceilings["scattered_row_write"], 4)
        if "gather_sum" in ceilings:
            ceilings["combine_frac_of_gather_sum"] = round(
                gbs("combine", nbytes["combine"]) / ceilings["gather_sum"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on the same workload")
        host = {
            "x": x.view(torch.int16).cpu().numpy().view(np.uint16),
            "expert_out": expert_out.view(torch.int16).cpu().numpy().view(np.uint16),
            "g_result": g_result.view(torch.int16).cpu().numpy().view(np.uint16),
            "g_recv": g_recv.view(torch.int16).cpu().numpy().view(np.uint16),
            "g_recv_w": g_recv_w.cpu().numpy(),
        }
        import oracle
        oracle.build()
        default_threads = oracle.set_threads(0)
        td, tc, n, spent, used = cpu_baseline(cfg, r, host, cap, args.cpu_budget, 0)
        td1, tc1, n1, spent1, _ = cpu_baseline(cfg, r, host, cap, args.cpu_budget, 1)
        oracle.set_threads(default_threads)
        cpu = {"value": round(pair_bytes / (td + tc) / 1e9, 3), "unit": "GB/s",
               "cores": used, "kind": "oracle",
               "sample": f"{n} whole step(s) of the {cfg.name} workload (all five ops, "
                         f"same inputs) by the C oracle with its row and token loops on "
                         f"{used} OpenMP threads, {spent:.1f} s; dispatch {td * 1e3:.1f} ms, "
                         f"combine {tc * 1e3:.1f} ms per step",
               "single_thread": {"value": round(pair_bytes / (td1 + tc1) / 1e9, 3),
                                 "unit": "GB/s", "cores": 1,
                                 "sample": f"{n1} whole step(s), {spent1:.1f} s; dispatch "
                                           f"{td1 * 1e3:.1f} ms, combine {tc1 * 1e3:.1f} ms"},
               "host_cpu_count": os.cpu_count()}

    line = {
        "metric": "dispatch+combine HBM GB/s (% of MI355X peak) and tokens/s, 1 GPU",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: T={T} H={H} E={E} topk={K} alignment={A} "
                               f"routing={cfg.routing} cap={cap}",
                   "global_batch": T, "parallelism": "none (one GPU's share)",
                   "masked_routes": not dense},
        "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(T / pair_s, 1),
        "value_is": args.headline,
        "warm": warm,
        "cold": cold,
        "ops": {op: {"avg_us": round(avg[op] * 1e3, 2), "median_us": round(med[op] * 1e3, 2),
                     "p10_us": round(p10[op] * 1e3, 2), "p90_us": round(p90[op] * 1e3, 2),
                     "algorithmic_bytes": nbytes[op],
                     "GBps": round(gbs(op, nbytes[op]), 1) if op != "prepare" else None}
                for op in STEP_OPS},
        "ops_outside_step": {op: {"avg_us": round(avg[op] * 1e3, 2),
                                  "median_us": round(med[op] * 1e3, 2),
                                  "p10_us": round(p10[op] * 1e3, 2),
                                  "p90_us": round(p90[op] * 1e3, 2),
                                  "algorithmic_bytes": nb,
                                  "GBps": round(gbs(op, nb), 1)}
                             for op, nb in extra.items()},
        "routing": {"R": nbytes["_R"], "P": nbytes["_P"], "total": nbytes["_total"],
                    "T_act": nbytes["_T_act"]},
        "roofline": roofline,
        "ceilings": ceilings,
        "cpu_baseline": cpu,
        **({"graph": graph} if graph is not None else {}),
        "kernel_source_hash": src_hash,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
