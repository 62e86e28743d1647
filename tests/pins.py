"""Property checkers for routing maps and payloads.

Each checker returns a list of human-readable violations (empty = pass). They
encode what the definition of prepare and dispatch fixes independently of any
implementation: the histogram, the aligned exclusive scan, the slot map being
a stable permutation of the valid routes, and pads at the segment ends.
"""
from __future__ import annotations

import numpy as np


def check_prepare(topk_idx, E, A, cap, counts, offsets, slot, row_src, status):
    errs = []
    idx = np.asarray(topk_idx, np.int64).reshape(-1)
    counts = np.asarray(counts, np.int64)
    offsets = np.asarray(offsets, np.int64)
    slot = np.asarray(slot, np.int64).reshape(-1)
    valid = (idx >= 0) & (idx < E)
    want_counts = np.bincount(idx[valid], minlength=E)
    if not np.array_equal(counts, want_counts):
        errs.append("counts differ from the histogram of valid ids")
    if offsets[0] != 0:
        errs.append("offsets[0] != 0")
    seg = np.diff(offsets)
    if (seg % A != 0).any():
        errs.append("a segment length is not a multiple of the alignment")
    if (seg < counts).any() or (seg - counts >= A).any():
        errs.append("a segment is not its count rounded up to the alignment")
    total = int(offsets[-1])
    bad = ((idx != -1) & ~valid).any()
    want_status = (1 if bad else 0) | (2 if total > cap else 0)
    if int(status) != want_status:
        errs.append(f"status {status} != {want_status}")
    if (slot[~valid] != -1).any():
        errs.append("a masked or bad route has a slot")
    live = min(total, cap)
    row_src = np.asarray(row_src, np.int64)[:live]
    vs = np.nonzero(valid)[0]
    e_of = idx[vs]
    for e in range(E):
        routes = vs[e_of == e]
        lo = offsets[e]
        want = lo + np.arange(len(routes))
        keep = want < cap
        if not np.array_equal(slot[routes[keep]], want[keep]):
            errs.append(f"expert {e}: slots are not the segment start plus the stable rank")
            break
        if (slot[routes[~keep]] != -1).any():
            errs.append(f"expert {e}: a route past the capacity kept a slot")
            break
    # row_src is the inverse of slot on the valid rows, -1 on pads.
    held = slot[slot >= 0]
    if len(np.unique(held)) != len(held):
        errs.append("two routes share a received row")
    if len(held) and (held.max() >= live or len(row_src) != live):
        errs.append("a slot lies past the live rows")
        return errs
    inv = np.full(live, -1, np.int64)
    inv[held] = np.nonzero(slot >= 0)[0]
    if not np.array_equal(row_src, inv):
        errs.append("row_src is not the inverse of slot with -1 pads")
    return errs


def check_pads_at_segment_end(offsets, counts, row_src, cap):
    errs = []
    offsets = np.asarray(offsets, np.int64)
    for e in range(len(counts)):
        lo, hi = offsets[e], min(offsets[e + 1], cap)
        body = row_src[lo:min(lo + counts[e], cap)]
        tail = row_src[min(lo + counts[e], cap):hi]
        if (body < 0).any() or (tail != -1).any():
            errs.append(f"expert {e}: pad rows are not at the end of the segment")
            break
        if len(body) > 1 and (np.diff(body) <= 0).any():
            errs.append(f"expert {e}: rows are not in ascending route order")
            break
    return errs


def dot_f64(a, b):
    return float(np.dot(np.asarray(a, np.float64).reshape(-1),
                        np.asarray(b, np.float64).reshape(-1)))
