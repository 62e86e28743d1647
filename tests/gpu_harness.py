"""Run the five ops on the GPU through the C ABI and compare with the oracle.

Every output buffer is pre-filled with a canary so that writes outside the
documented rows show up. Comparisons are on raw bits (uint16 for bf16,
uint32 for fp32): NaN payloads, signed zeros and subnormals must all match.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import combine_ep_prepare_amd as ep
import oracle

CANARY_BF16 = 0xBEEF
CANARY_F32 = np.float32(-1234.5)   # exact in fp32, never produced by the ops


def log(msg: str):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def dev_bf16(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16)


def host_bf16(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


def host_f32(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def bits32(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def _fill_bf16(rows, H):
    t = torch.empty((rows, H), dtype=torch.int16, device="cuda")
    t.fill_(np.array([CANARY_BF16], np.uint16).view(np.int16)[0].item())
    return t.view(torch.bfloat16)


def _fill_f32(n):
    return torch.full((n,), float(CANARY_F32), dtype=torch.float32, device="cuda")


class GpuRun:
    """One handle: prepare, then any of the payload ops."""

    def __init__(self, topk_idx: np.ndarray, E: int, A: int, H: int, cap: int,
                 stream=None, prepare_dtype="bf16"):
        T, K = topk_idx.shape
        self.layout = ep.Layout(T, K, E, A, H, cap)
        # prepare sizes the run chunks from its layout's row: a layout of
        # another payload type gives another chunk size, same results
        self.prepare_layout = ep.Layout(T, K, E, A, H, cap, dtype=prepare_dtype)
        self.T, self.K, self.E, self.A, self.H, self.cap = T, K, E, A, H, cap
        self.stream = stream
        self.handle = ep.new_handle(self.layout)
        self.idx = torch.from_numpy(np.ascontiguousarray(topk_idx, np.int64)).to("cuda")
        self.counts = torch.full((E,), -5, dtype=torch.int32, device="cuda")
        self.offsets = torch.full((E + 1,), -5, dtype=torch.int32, device="cuda")

    def prepare(self, with_offsets=True):
        ep.prepare(self.prepare_layout, self.idx, self.counts, self.handle,
                   self.offsets if with_offsets else None, stream=self.stream)

    def maps(self) -> dict:
        m = ep.handle_maps(self.layout, self.handle)
        torch.cuda.synchronize()
        return {k: v.cpu().numpy() for k, v in m.items()}

    def status(self) -> int:
        return ep.read_status(self.handle, stream=self.stream)

    def dispatch(self, x: torch.Tensor, w: torch.Tensor | None):
        recv = _fill_bf16(self.cap, self.H)
        recv_w = _fill_f32(self.cap) if w is not None else None
        ep.dispatch(self.layout, self.handle, x, w, recv, recv_w, stream=self.stream)
        return recv, recv_w

    def combine(self, rows: torch.Tensor):
        out = _fill_bf16(self.T, self.H)
        ep.combine(self.layout, self.handle, rows, out, stream=self.stream)
        return out

    def combine_bwd(self, g: torch.Tensor):
        out = _fill_bf16(self.cap, self.H)
        ep.combine_bwd(self.layout, self.handle, g, out, stream=self.stream)
        return out

    def dispatch_bwd(self, g: torch.Tensor, g_w: torch.Tensor | None, want_w=True):
        gt = _fill_bf16(self.T, self.H)
        gw = _fill_f32(self.T * self.K).view(self.T, self.K) if want_w else None
        ep.dispatch_bwd(self.layout, self.handle, g, g_w, gt, gw, stream=self.stream)
        return gt, gw


def wbwd_gamma(H: int, dt: str = "bf16") -> float:
    """gamma_n = n u / (1 - n u) for the weighted backward's weight gradient:
    each product passes through at most n = N + P + 5 fp32 roundings, N the
    elements of a 16-byte vector and P = ceil(H * elem / 1024) the row's
    64-lane pieces (a fused multiply-add chain of N per lane, six butterfly
    adds per piece, P - 1 adds over the pieces), the bound ep.h states."""
    elem = 4 if dt == "fp32" else 2
    n = 16 // elem + -(-(H * elem) // 1024) + 5
    u = 2.0 ** -24
    return n * u / (1 - n * u)


def check_run_entries(m: dict, slot: np.ndarray, topk_idx: np.ndarray, E: int):
    """The run entries against their definition and the oracle's slot map:
    chunks of run_units * 512 routes, chunk c in list c mod 8 after the
    stream's earlier chunks; each chunk's routes that hold a row in ascending
    row order, then (-1, -1) for each valid route dropped past the capacity;
    each list's length in stream_live."""
    runs, live, ru = m["runs"], m["stream_live"], int(m["run_units"][0])
    assert ru in (1, 2, 4)
    CK = ru * 512
    routes = slot.size
    ids = topk_idx.reshape(-1)
    pos = np.zeros(8, np.int64)
    for c in range((routes + CK - 1) // CK):
        s0, s1 = c * CK, min((c + 1) * CK, routes)
        x = c % 8
        nvalid = int(((ids[s0:s1] >= 0) & (ids[s0:s1] < E)).sum())
        e = runs[x, pos[x]:pos[x] + nvalid]
        want = np.arange(s0, s1)[slot[s0:s1] >= 0]
        n = len(want)
        assert (e[n:] == -1).all(), f"chunk {c}: empty entries"
        got_rows, got_routes = e[:n, 0], e[:n, 1]
        assert (np.diff(got_rows) > 0).all(), f"chunk {c}: rows not ascending"
        assert np.array_equal(np.sort(got_routes), want), f"chunk {c}: routes"
        assert np.array_equal(slot[got_routes], got_rows), f"chunk {c}: rows of routes"
        pos[x] += nvalid
    assert np.array_equal(live, pos), "stream list lengths"


def check_prepare(run: GpuRun, p: oracle.Prepared):
    m = run.maps()
    counts = run.counts.cpu().numpy()
    offsets = run.offsets.cpu().numpy()
    assert np.array_equal(counts, p.counts), "token_counts"
    assert np.array_equal(offsets, p.offsets), "expert_offsets"
    assert np.array_equal(m["counts"], p.counts), "handle counts"
    assert np.array_equal(m["offsets"], p.offsets), "handle offsets"
    assert np.array_equal(m["slot"], p.slot), "slot map"
    assert np.array_equal(m["row_src"][:p.live], p.row_src[:p.live]), "row_src"
    check_run_entries(m, p.slot, run.idx.cpu().numpy(), run.E)
    assert run.status() == p.status, "status"


def check_all_ops(run: GpuRun, p: oracle.Prepared, x: np.ndarray, w: np.ndarray | None,
                  rows: np.ndarray, g_result: np.ndarray, g_recv: np.ndarray,
                  g_recv_w: np.ndarray | None, label: str = "",
                  dev: dict | None = None):
    """Compare every op with the oracle, bit for bit, canaries included.

    ``dev`` may carry device copies of the payloads (already resident) so
    that large inputs are not uploaded twice."""
    dev = dev or {}
    H, cap, live = run.H, run.cap, p.live
    xd = dev.get("x", None)
    xd = dev_bf16(x) if xd is None else xd
    wd = None if w is None else dev_f32(w)
    log(f"{label}: dispatch")
    recv, recv_w = run.dispatch(xd, wd)
    o_recv, o_recv_w = oracle.dispatch(p, x, w, recv_init=np.full((cap, H), CANARY_BF16,
                                                                 np.uint16),
                                       recv_w_init=np.full(cap, CANARY_F32, np.float32)
                                       if w is not None else None)
    assert np.array_equal(host_bf16(recv), o_recv), f"{label}: dispatch rows"
    if w is not None:
        assert np.array_equal(bits32(host_f32(recv_w)), bits32(o_recv_w)), \
            f"{label}: dispatch weights"
    del recv, recv_w

    log(f"{label}: combine")
    rd = dev.get("rows", None)
    rd = dev_bf16(rows) if rd is None else rd
    out = run.combine(rd)
    assert np.array_equal(host_bf16(out), oracle.combine(p, rows)), f"{label}: combine"
    del out, rd

    log(f"{label}: combine_bwd")
    gd = dev.get("g_result", None)
    gd = dev_bf16(g_result) if gd is None else gd
    gb = run.combine_bwd(gd)
    o_gb = oracle.combine_bwd(p, g_result, init=np.full((cap, H), CANARY_BF16, np.uint16))
    assert np.array_equal(host_bf16(gb), o_gb), f"{label}: combine_bwd"
    del gb, gd

    log(f"{label}: dispatch_bwd")
    Gd = dev.get("g_recv", None)
    Gd = dev_bf16(g_recv) if Gd is None else Gd
    gwd = None if g_recv_w is None else dev_f32(g_recv_w)
    gt, gw = run.dispatch_bwd(Gd, gwd)
    o_gt, o_gw = oracle.dispatch_bwd(p, g_recv, g_recv_w)
    assert np.array_equal(host_bf16(gt), o_gt), f"{label}: dispatch_bwd tokens"
    assert np.array_equal(bits32(host_f32(gw)), bits32(o_gw)), f"{label}: dispatch_bwd weights"
    assert run.status() == p.status, f"{label}: status after payload ops"
