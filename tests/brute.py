"""Brute-force NumPy/PyTorch models of the five ops, for tiny inputs only.

These are a second, independent formulation used to pin the C oracle: prepare
is a histogram (``np.bincount``) plus a stable argsort by expert id, dispatch
is written as a scatter from routes (the oracle writes a gather over rows),
and combine accumulates whole columns in NumPy float32 with PyTorch's own
fp32 -> bf16 conversion for the final rounding.
"""
from __future__ import annotations

import numpy as np
import torch


def f32_to_bf16_torch(a: np.ndarray) -> np.ndarray:
    """PyTorch's fp32 -> bf16 (round to nearest even); NaNs are then set to
    the canonical quiet NaN 0x7FC0, the reading both implementations follow."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    t = torch.from_numpy(a)
    out = t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    out[np.isnan(a)] = 0x7FC0
    return out


def bf16_to_f32_np(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f16_to_f32_np(b: np.ndarray) -> np.ndarray:
    """NumPy's binary16 -> binary32 (exact)."""
    return np.ascontiguousarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)


def f32_to_f16_np(a: np.ndarray) -> np.ndarray:
    """NumPy's binary32 -> binary16 (round to nearest even); NaNs then set to
    the canonical quiet NaN 0x7E00."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    with np.errstate(over="ignore"):
        out = a.astype(np.float16).view(np.uint16).copy()
    out[np.isnan(a)] = 0x7E00
    return out


def f32_canon_np(a: np.ndarray) -> np.ndarray:
    out = np.array(a, dtype=np.float32, copy=True)
    out.view(np.uint32)[np.isnan(out)] = 0x7FC00000
    return out


# payload type -> (widen to fp32, round fp32 once to the type)
CODECS = {
    "bf16": (bf16_to_f32_np, f32_to_bf16_torch),
    "fp16": (f16_to_f32_np, f32_to_f16_np),
    "fp32": (lambda a: np.asarray(a, dtype=np.float32), f32_canon_np),
}


def prepare(topk_idx: np.ndarray, E: int, A: int, cap: int):
    idx = np.asarray(topk_idx, dtype=np.int64)
    T, K = idx.shape
    flat = idx.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    bad = bool(((flat != -1) & ~valid).any())
    counts = np.bincount(flat[valid], minlength=E).astype(np.int64)
    padded = -(-counts // A) * A
    offsets = np.concatenate([[0], np.cumsum(padded)]).astype(np.int64)
    total = int(offsets[-1])
    key = np.where(valid, flat, E)          # masked routes sort after every expert
    order = np.argsort(key, kind="stable")
    slot = np.full(T * K, -1, np.int64)
    starts = np.concatenate([[0], np.cumsum(counts)])
    for e in range(E):
        routes = order[starts[e]:starts[e + 1]]
        slot[routes] = offsets[e] + np.arange(len(routes))
    overflow = total > cap
    slot[slot >= cap] = -1
    live = min(total, cap)
    row_src = np.full(live, -1, np.int64)
    vs = np.nonzero(slot >= 0)[0]
    row_src[slot[vs]] = vs
    status = (1 if bad else 0) | (2 if overflow else 0)
    return dict(counts=counts, offsets=offsets, slot=slot, row_src=row_src,
                status=status, total=total, live=live)


def dispatch(prep, x: np.ndarray, w: np.ndarray | None, K: int, cap: int):
    T, H = x.shape
    recv = np.zeros((cap, H), x.dtype)
    recv_w = np.zeros(cap, np.float32)
    for s, r in enumerate(prep["slot"]):
        if r >= 0:
            recv[r] = x[s // K]
            if w is not None:
                recv_w[r] = w.reshape(-1)[s]
    return recv, recv_w


def combine(prep, rows: np.ndarray, T: int, K: int, dtype: str = "bf16"):
    widen, narrow = CODECS[dtype]
    H = rows.shape[1]
    slot = prep["slot"].reshape(T, K)
    acc = np.zeros((T, H), np.float32)
    have = np.zeros(T, bool)
    for k in range(K):
        r = slot[:, k]
        ok = r >= 0
        v = widen(rows[np.where(ok, r, 0)])
        first = ok & ~have
        later = ok & have
        acc[first] = v[first]
        with np.errstate(over="ignore", invalid="ignore"):
            acc[later] = acc[later] + v[later]
        have |= ok
    out = narrow(acc)
    out[~have] = 0
    return out


def dispatch_bwd_weights(prep, g_recv_w: np.ndarray | None, T: int, K: int):
    gw = np.zeros(T * K, np.float32)
    if g_recv_w is not None:
        for s, r in enumerate(prep["slot"]):
            if r >= 0:
                gw[s] = g_recv_w[r]
    return gw.reshape(T, K)
