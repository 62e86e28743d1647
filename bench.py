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
bounded sample of the same workload on this host. The fused weighted combine
and its backward are timed after the step, the same way, and reported beside
it ("ops_outside_step").

    python bench.py [--steps K] [--warmup W] [--workload dsv3] [--no-cpu-baseline]
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


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(T, K, E, H, topk_idx, counts_np, offsets_np):
    """Bytes each op must move at minimum (each row once).

    B = 2H bytes per bf16 row, R valid routes, P pad rows, T_act tokens with
    at least one valid route.
      dispatch      T_act*B + (R+P)*B + 4R + 8(R+P)   rows, weights in/out, row map
      combine       R*B + T*B + 4TK                   rows in/out, slot map
      combine_bwd   T_act*B + (R+P)*B + 4(R+P)        rows in/out, row map
      dispatch_bwd  R*B + 4R + T*B + 8TK              rows in/out, weights, slot map
      prepare       8TK + 4TK + 4(R+P) + 8E           ids, slots, row map, counts
      combine_weighted      R*B + 4R + T*B + 4TK      rows and weights in, rows out, slot map
      combine_weighted_bwd  T_act*B + R*B + 4R + (R+P)*B + 4(R+P) + 4TK + 4P
                            grads in, expert rows and weights in, row and weight
                            grads out, slot map, pad-row list
    """
    import numpy as np
    B = 2 * H
    R = int(counts_np.sum())
    total = int(offsets_np[-1])
    P = total - R
    T_act = int((topk_idx >= 0).any(axis=1).sum()) if T else 0
    return {
        "dispatch": T_act * B + (R + P) * B + 4 * R + 8 * (R + P),
        "combine": R * B + T * B + 4 * T * K,
        "combine_bwd": T_act * B + (R + P) * B + 4 * (R + P),
        "dispatch_bwd": R * B + 4 * R + T * B + 8 * T * K,
        "prepare": 8 * T * K + 4 * T * K + 4 * (R + P) + 8 * E,
        "combine_weighted": R * B + 4 * R + T * B + 4 * T * K,
        "combine_weighted_bwd": (T_act * B + R * B + 4 * R + (R + P) * B + 4 * (R + P)
                                 + 4 * T * K + 4 * P),
        "_R": R, "_P": P, "_T_act": T_act, "_total": total,
    }


def _pmc_path(op: str, workload: str) -> str:
    return os.path.join(PROFILE_DIR, f"{KERNEL_OF_OP[op]}_{op}_{workload}_pmc.txt")


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


def _read_csv_rows(directory: str, suffix: str):
    import csv
    import glob
    rows = []
    for path in sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True)):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


KERNEL_OF_OP = {"dispatch": "scatter_rows_kernel", "combine_bwd": "scatter_rows_kernel",
                "combine": "reduce_rows_kernel", "dispatch_bwd": "reduce_rows_kernel",
                "combine_weighted": "reduce_rows_kernel",
                "combine_weighted_bwd": "weighted_bwd_kernel"}


def op_sequence(names):
    """Attribute each payload-kernel dispatch (demangled names, in dispatch
    order) to its op. Within a step the unweighted scatter runs for dispatch,
    then combine_bwd; the unweighted reduce for combine, then dispatch_bwd.
    The weighted reduce (template flag true) and the weighted backward kernel
    each serve one op. Other kernels map to None."""
    out = []
    n_scatter = n_reduce = 0
    for name in names:
        if "scatter_rows_kernel" in name:
            out.append(("dispatch", "combine_bwd")[n_scatter % 2])
            n_scatter += 1
        elif "reduce_rows_kernel" in name and "true" in name:
            out.append("combine_weighted")
        elif "reduce_rows_kernel" in name:
            out.append(("combine", "dispatch_bwd")[n_reduce % 2])
            n_reduce += 1
        elif "weighted_bwd_kernel" in name:
            out.append("combine_weighted_bwd")
        else:
            out.append(None)
    return out


def summarize_pmc(fetch_dir: str, write_dir: str, workload: str, copy_mib: int,
                  out_dir: str = PROFILE_DIR):
    """Turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then
    WRITE_SIZE, both with --calibration-copy-mib) into per-op HBM bytes.

    Each counter is scaled by what it reads for the plain copy of known size
    (PyTorch's elementwise copy kernel, the largest dispatch whose name holds
    "copy"), so the result is in true bytes. Dispatches of our two payload
    kernels are attributed to ops by their order inside each step: scatter
    (dispatch), reduce (combine), scatter (combine_bwd), reduce (dispatch_bwd).
    """
    import numpy as np
    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _read_csv_rows(d, "counter_collection.csv")
                if r.get("Counter_Name") == counter]
        rows.sort(key=lambda r: int(r.get("Dispatch_Id", 0)))
        # the calibration copy is a plain device-to-device copy of copy_mib
        # MiB (PyTorch hands it to the runtime's copyBuffer kernel)
        calib = [r for r in rows if "copybuffer" in r["Kernel_Name"].lower()
                 and float(r["Counter_Value"]) > copy_mib * 1024.0 / 8]
        if not calib:
            raise SystemExit(f"no calibration copy found for {counter} in {d}")
        expected_kib = copy_mib * 1024.0
        factor = float(np.median([float(r["Counter_Value"]) for r in calib])) / expected_kib
        # the timed steps follow the calibration copy; the one dispatch made
        # before it (to build the expert outputs) is left out
        last_copy = max(int(r.get("Dispatch_Id", 0)) for r in calib)
        seq = [(r["Kernel_Name"], float(r["Counter_Value"])) for r in rows
               if int(r.get("Dispatch_Id", 0)) > last_copy]
        per_op = {op: [] for op in KERNEL_OF_OP}
        for (name, kib), op in zip(seq, op_sequence([nm for nm, _ in seq])):
            if op is not None:
                per_op[op].append(kib / factor * 1024.0)
        res[counter] = {"factor": factor,
                        "per_op_bytes": {op: float(np.median(v)) for op, v in per_op.items() if v}}
    out = {"workload": workload, "kernel_source_hash": kernel_source_hash(),
           "calibration": {"copy_mib": copy_mib,
                           "fetch_factor": res["FETCH_SIZE"]["factor"],
                           "write_factor": res["WRITE_SIZE"]["factor"]}}
    cmd = ("cd /tmp && export TMPDIR=/tmp && timeout -s KILL 120 rocprofv3 --pmc <COUNTER> "
           "-d <dir> -o <name> --output-format csv -- python3 bench.py --workload "
           f"{workload} --steps 3 --warmup 1 --no-cpu-baseline --calibration-copy-mib {copy_mib}"
           "   (once with FETCH_SIZE, once with WRITE_SIZE); then python bench.py "
           f"--summarize-pmc <fetch dir> <write dir> --workload {workload} "
           f"--calibration-copy-mib {copy_mib}")
    for op in KERNEL_OF_OP:
        fb = res["FETCH_SIZE"]["per_op_bytes"].get(op)
        wb = res["WRITE_SIZE"]["per_op_bytes"].get(op)
        if fb is None or wb is None:
            continue
        summary = dict(out)
        summary.update({"op": op, "kernel": KERNEL_OF_OP[op], "fetch_bytes_per_launch": fb,
                        "write_bytes_per_launch": wb, "hbm_bytes_per_launch": fb + wb})
        path = _pmc_path(op, workload)
        with open(path, "w") as f:
            f.write(f"# HBM traffic of {KERNEL_OF_OP[op]} ({op}), workload {workload}\n")
            f.write(f"# command: {cmd}\n")
            f.write(f"# FETCH_SIZE scale {out['calibration']['fetch_factor']:.4f}, WRITE_SIZE "
                    f"scale {out['calibration']['write_factor']:.4f} (counter / true bytes of "
                    f"a {copy_mib} MiB device copy in the same run)\n")
            f.write(f"# per launch (median over the timed steps): fetch {fb / 1e6:.1f} MB, "
                    f"write {wb / 1e6:.1f} MB, total {(fb + wb) / 1e6:.1f} MB\n")
            f.write("JSON: " + json.dumps(summary) + "\n")
        print(f"{path}: fetch {fb / 1e6:.1f} MB write {wb / 1e6:.1f} MB", flush=True)


def summarize_trace(trace_dir: str, workload: str, steps: int, warmup: int,
                    out_dir: str = PROFILE_DIR):
    """profiles/ep_kernels_<workload>_kernel_stats.txt from a rocprofv3
    --kernel-trace --stats run of this script."""
    rows = _read_csv_rows(trace_dir, "kernel_stats.csv")
    path = os.path.join(out_dir, f"ep_kernels_{workload}_kernel_stats.txt")
    cmd = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -d <dir> -o "
           f"trace --output-format csv -- python3 bench.py --workload {workload} --steps "
           f"{steps} --warmup {warmup} --no-cpu-baseline")
    with open(path, "w") as f:
        f.write(f"# rocprofv3 kernel statistics, workload {workload}\n")
        f.write(f"# command: {cmd}\n")
        f.write(f"# kernel source hash {kernel_source_hash()}\n")
        f.write(f"{'kernel':60s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} "
                f"{'share%':>7s}\n")
        for r in rows:
            name = r["Name"]
            short = name.split("(")[0].replace("void ", "")
            f.write(f"{short[:60]:60s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} "
                    f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} "
                    f"{float(r['Percentage']):7.2f}\n")
    print(path, flush=True)


def cpu_baseline(cfg, r, host, cap, budget_s=12.0):
    """The oracle as it stands, single-threaded, on the same inputs: whole
    steps repeated until the time budget is spent (at least one)."""
    import numpy as np
    import oracle
    oracle.build()
    t_d = t_c = 0.0
    n = 0
    start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
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
    return t_d / n, t_c / n, n, time.perf_counter() - start


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra-ops", action="store_true",
                    help="skip timing the weighted combine and its backward")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="run a plain device copy of this size first (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/*_pmc.txt from two rocprofv3 counter runs")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="write profiles/*_kernel_stats.txt from a rocprofv3 --stats run")
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
        print("bench.py measures one GPU's share of the path; runs on more than one GPU "
              "are not part of this build (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

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

    # The experts' stand-in: expert_out = bf16(recv * recv_topk_weights),
    # computed once outside the timed region (the caller's pre-multiply).
    ep.prepare(L, idx, counts, handle, offsets)
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

    ops = ["prepare", "dispatch", "combine", "combine_bwd", "dispatch_bwd"]
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        ep.prepare(L, idx, counts, handle, offsets)
        if ev is not None:
            ev[1].record(stream)
        ep.dispatch(L, handle, x, w, recv, recv_w)
        if ev is not None:
            ev[2].record(stream)
        ep.combine(L, handle, expert_out, result)
        if ev is not None:
            ev[3].record(stream)
        ep.combine_bwd(L, handle, g_result, g_exp)
        if ev is not None:
            ev[4].record(stream)
        ep.dispatch_bwd(L, handle, g_recv, g_recv_w, g_tok, g_w)
        if ev is not None:
            ev[5].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert ep.read_status(handle) == 0, "unexpected status bits"

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    per_op_ms = {op: [] for op in ops}
    for ev in events:
        for j, op in enumerate(ops):
            per_op_ms[op].append(ev[j].elapsed_time(ev[j + 1]))
    avg = {op: float(np.mean(v)) for op, v in per_op_ms.items()}
    med = {op: float(np.median(v)) for op, v in per_op_ms.items()}

    # The fused weighted combine and its backward: not part of the step (the
    # step's combine is the unweighted one), timed the same way after it.
    extra_ops = [] if args.no_extra_ops else ["combine_weighted", "combine_weighted_bwd"]
    if extra_ops:
        result_w = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
        g_rows_w = torch.empty(cap, H, dtype=torch.bfloat16, device=dev)
        g_recv_w2 = torch.empty(cap, dtype=torch.float32, device=dev)

        def extra(ev=None):
            if ev is not None:
                ev[0].record(stream)
            ep.combine_weighted(L, handle, recv, recv_w, result_w)
            if ev is not None:
                ev[1].record(stream)
            ep.combine_weighted_bwd(L, handle, g_result, recv, recv_w, g_rows_w, g_recv_w2)
            if ev is not None:
                ev[2].record(stream)

        for _ in range(args.warmup):
            extra()
        xev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            extra(xev[i])
        torch.cuda.synchronize()
        assert ep.read_status(handle) == 0, "unexpected status bits"
        for j, op in enumerate(extra_ops):
            v = [ev[j].elapsed_time(ev[j + 1]) for ev in xev]
            avg[op] = float(np.mean(v))
            med[op] = float(np.median(v))

    def gbs(op):
        return nbytes[op] / (avg[op] * 1e-3) / 1e9

    pair_bytes = nbytes["dispatch"] + nbytes["combine"]
    pair_s = (avg["dispatch"] + avg["combine"]) * 1e-3
    value = pair_bytes / pair_s / 1e9
    dominant = max(("dispatch", "combine", "combine_bwd", "dispatch_bwd"),
                   key=lambda op: avg[op])
    kernel_of = KERNEL_OF_OP
    src_hash = kernel_source_hash()
    traffic = load_traffic(dominant, cfg.name, src_hash)
    achieved = gbs(dominant)
    roofline = {"bound": "hbm", "kernel": f"{kernel_of[dominant]} ({dominant})",
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic,
                "algorithmic_bytes_per_launch": nbytes[dominant],
                "avg_launch_us": round(avg[dominant] * 1e3, 2)}

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
        td, tc, n, spent = cpu_baseline(cfg, r, host, cap, args.cpu_budget)
        cpu = {"value": round(pair_bytes / (td + tc) / 1e9, 3), "unit": "GB/s",
               "cores": 1, "kind": "oracle",
               "sample": f"{n} whole step(s) of the {cfg.name} workload (all five ops, "
                         f"same inputs) by the single-threaded C oracle, {spent:.1f} s; "
                         f"dispatch {td * 1e3:.1f} ms, combine {tc * 1e3:.1f} ms per step",
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
                   "global_batch": T, "parallelism": "none (one GPU's share)"},
        "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(T / pair_s, 1),
        "ops": {op: {"avg_us": round(avg[op] * 1e3, 2), "median_us": round(med[op] * 1e3, 2),
                     "algorithmic_bytes": nbytes[op],
                     "GBps": round(gbs(op), 1) if op != "prepare" else None}
                for op in ops},
        "ops_outside_step": {op: {"avg_us": round(avg[op] * 1e3, 2),
                                  "median_us": round(med[op] * 1e3, 2),
                                  "algorithmic_bytes": nbytes[op],
                                  "GBps": round(gbs(op), 1)}
                             for op in extra_ops},
        "routing": {"R": nbytes["_R"], "P": nbytes["_P"], "total": nbytes["_total"],
                    "T_act": nbytes["_T_act"]},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernel_source_hash": src_hash,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
