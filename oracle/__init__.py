"""NumPy-facing wrapper of the CPU oracle (``oracle/ep_oracle.c``).

Test infrastructure: only the tests, the smoke check and the benchmark's
CPU-baseline leg use this package. The HIP library never imports it.

The C file is compiled with gcc into ``oracle/libep_oracle.so`` by
:func:`build`; every function here only marshals NumPy arrays into it.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ep_oracle.c")
_LIB = os.path.join(_HERE, "libep_oracle.so")

STATUS_BAD_EXPERT = 1
STATUS_OVERFLOW = 2

# Plain scalar C: no fast-math, no contraction, IEEE binary32 via SSE. OpenMP
# shares the loops over received rows and over tokens among threads (see
# set_threads); every result bit is the same on any thread count.
CFLAGS = ["-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-msse2", "-mfpmath=sse", "-fopenmp", "-Wall", "-Werror"]


def build() -> str:
    """Compile the oracle with gcc (always rebuilds)."""
    tmp = _LIB + ".tmp"
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = C.CDLL(_LIB)
        i64, i32, u32p, vp = C.c_int64, C.c_int32, C.POINTER(C.c_uint32), C.c_void_p
        lib.ep_oracle_prepare.argtypes = [i64, i32, i32, i32, i64, vp, vp, vp, vp, vp, u32p]
        lib.ep_oracle_prepare.restype = C.c_int
        lib.ep_oracle_dispatch.argtypes = [i64, i32, i64, C.c_int, C.c_int, C.c_int, i64,
                                           i64, vp, vp, vp, vp, vp]
        lib.ep_oracle_dispatch.restype = C.c_int
        lib.ep_oracle_combine_bwd.argtypes = [i64, i32, i64, C.c_int, C.c_int, C.c_int, i64,
                                              i64, vp, vp, vp]
        lib.ep_oracle_combine_bwd.restype = C.c_int
        lib.ep_oracle_combine.argtypes = [i64, i32, i64, C.c_int, vp, vp, vp]
        lib.ep_oracle_combine.restype = C.c_int
        lib.ep_oracle_dispatch_bwd.argtypes = [i64, i32, i64, C.c_int, vp, vp, vp, vp, vp]
        lib.ep_oracle_dispatch_bwd.restype = C.c_int
        lib.ep_oracle_combine_weighted.argtypes = [i64, i32, i64, C.c_int, vp, vp, vp, vp]
        lib.ep_oracle_combine_weighted.restype = C.c_int
        lib.ep_oracle_combine_weighted_bwd.argtypes = [i64, i32, i64, C.c_int, C.c_int,
                                                       C.c_int, i64, i64, vp, vp, vp, vp, vp,
                                                       vp, vp]
        lib.ep_oracle_combine_weighted_bwd.restype = C.c_int
        lib.ep_oracle_f16_to_f32.argtypes = [C.c_uint16]
        lib.ep_oracle_f16_to_f32.restype = C.c_float
        lib.ep_oracle_f32_to_f16.argtypes = [C.c_float]
        lib.ep_oracle_f32_to_f16.restype = C.c_uint16
        lib.ep_oracle_f32_to_bf16.argtypes = [C.c_float]
        lib.ep_oracle_f32_to_bf16.restype = C.c_uint16
        lib.ep_oracle_bf16_to_f32.argtypes = [C.c_uint16]
        lib.ep_oracle_bf16_to_f32.restype = C.c_float
        lib.ep_oracle_recv_capacity_worst.argtypes = [i64, i32, i32, i32]
        lib.ep_oracle_recv_capacity_worst.restype = i64
        lib.ep_oracle_set_threads.argtypes = [C.c_int]
        lib.ep_oracle_set_threads.restype = C.c_int
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


@dataclass
class Prepared:
    counts: np.ndarray    # int32 [E]
    offsets: np.ndarray   # int32 [E+1]
    slot: np.ndarray      # int32 [T*K]
    row_src: np.ndarray   # int32 [cap]; rows >= min(total, cap) hold the fill value
    status: int
    T: int
    K: int
    E: int
    A: int
    cap: int

    @property
    def total(self) -> int:
        return int(self.offsets[-1])

    @property
    def live(self) -> int:
        return min(self.total, self.cap)


def set_threads(n: int = 0) -> int:
    """Threads the oracle's row and token loops use from now on (n >= 1), or
    none changed (n = 0); returns the count in force."""
    return int(_load().ep_oracle_set_threads(int(n)))


def recv_capacity_worst(T, K, E, A) -> int:
    return int(_load().ep_oracle_recv_capacity_worst(T, K, E, A))


def f32_to_bf16(f: float) -> int:
    return int(_load().ep_oracle_f32_to_bf16(C.c_float(f)))


def bf16_to_f32(h: int) -> float:
    return float(_load().ep_oracle_bf16_to_f32(C.c_uint16(h)))


def f32_to_f16(f: float) -> int:
    return int(_load().ep_oracle_f32_to_f16(C.c_float(f)))


def f16_to_f32(h: int) -> float:
    return float(_load().ep_oracle_f16_to_f32(C.c_uint16(h)))


# Payload types: name -> (code of the C oracle, NumPy storage type of a row
# element). bf16 and fp16 rows are held as their 16-bit patterns.
DTYPES = {"bf16": (0, np.uint16), "fp16": (1, np.uint16), "fp32": (2, np.float32)}


def _rows(a, dtype):
    return np.ascontiguousarray(a, dtype=DTYPES[dtype][1])


def prepare(topk_idx: np.ndarray, E: int, A: int, cap: int, fill: int = -7) -> Prepared:
    topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int64)
    T, K = topk_idx.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    slot = np.empty(max(T * K, 1), np.int32)
    row_src = np.full(max(cap, 1), fill, np.int32)
    st = C.c_uint32(0)
    rc = _load().ep_oracle_prepare(T, K, E, A, cap, _p(topk_idx), _p(counts), _p(offsets),
                                   _p(slot), _p(row_src), C.byref(st))
    _check(rc, "prepare")
    return Prepared(counts, offsets, slot[:T * K], row_src[:cap], int(st.value), T, K, E,
                    A, cap)


def dispatch(prep: Prepared, x: np.ndarray, w: np.ndarray | None,
             recv_init: np.ndarray | None = None, recv_w_init: np.ndarray | None = None,
             dtype: str = "bf16", fill_pads: bool = True, zero_tail: bool = False):
    """Returns (recv [cap,H], recv_w f32 [cap] or None). Rows past the live
    total (unless zero_tail) and pad rows when fill_pads is False keep the
    values of the ``*_init`` arrays (zeros if not given)."""
    x = _rows(x, dtype)
    T, H = x.shape
    st = DTYPES[dtype][1]
    recv = (np.zeros((prep.cap, H), st) if recv_init is None
            else np.array(recv_init, dtype=st, copy=True))
    recv_w = None
    if w is not None:
        w = np.ascontiguousarray(w, dtype=np.float32)
        recv_w = (np.zeros(prep.cap, np.float32) if recv_w_init is None
                  else np.array(recv_w_init, dtype=np.float32, copy=True))
    rc = _load().ep_oracle_dispatch(T, prep.K, H, DTYPES[dtype][0], int(fill_pads),
                                    int(zero_tail), prep.cap, prep.total, _p(prep.row_src),
                                    _p(x), _p(w), _p(recv), _p(recv_w))
    _check(rc, "dispatch")
    return recv, recv_w


def combine_bwd(prep: Prepared, g_result: np.ndarray, init: np.ndarray | None = None,
                dtype: str = "bf16", fill_pads: bool = True, zero_tail: bool = False):
    g_result = _rows(g_result, dtype)
    T, H = g_result.shape
    st = DTYPES[dtype][1]
    out = (np.zeros((prep.cap, H), st) if init is None
           else np.array(init, dtype=st, copy=True))
    rc = _load().ep_oracle_combine_bwd(T, prep.K, H, DTYPES[dtype][0], int(fill_pads),
                                       int(zero_tail), prep.cap, prep.total, _p(prep.row_src),
                                       _p(g_result), _p(out))
    _check(rc, "combine_bwd")
    return out


def combine(prep: Prepared, rows: np.ndarray, T: int | None = None, dtype: str = "bf16"):
    rows = _rows(rows, dtype)
    H = rows.shape[1]
    T = prep.T if T is None else T
    out = np.empty((T, H), DTYPES[dtype][1])
    rc = _load().ep_oracle_combine(T, prep.K, H, DTYPES[dtype][0], _p(prep.slot), _p(rows),
                                   _p(out))
    _check(rc, "combine")
    return out


def dispatch_bwd(prep: Prepared, g_recv: np.ndarray, g_recv_w: np.ndarray | None,
                 want_grad_w: bool = True, dtype: str = "bf16"):
    g_recv = _rows(g_recv, dtype)
    H = g_recv.shape[1]
    T, K = prep.T, prep.K
    gt = np.empty((T, H), DTYPES[dtype][1])
    gw = np.empty((T, K), np.float32) if want_grad_w else None
    if g_recv_w is not None:
        g_recv_w = np.ascontiguousarray(g_recv_w, dtype=np.float32)
    rc = _load().ep_oracle_dispatch_bwd(T, K, H, DTYPES[dtype][0], _p(prep.slot), _p(g_recv),
                                        _p(g_recv_w), _p(gt), _p(gw))
    _check(rc, "dispatch_bwd")
    return gt, gw


def combine_weighted(prep: Prepared, rows: np.ndarray, w: np.ndarray, T: int | None = None,
                     dtype: str = "bf16"):
    """[T,H]: sum over valid k (ascending) of w[r] * rows[r], first term a
    product, later terms fused multiply-adds, one rounding to the payload type."""
    rows = _rows(rows, dtype)
    w = np.ascontiguousarray(w, dtype=np.float32)
    H = rows.shape[1]
    T = prep.T if T is None else T
    out = np.empty((T, H), DTYPES[dtype][1])
    rc = _load().ep_oracle_combine_weighted(T, prep.K, H, DTYPES[dtype][0], _p(prep.slot),
                                            _p(rows), _p(w), _p(out))
    _check(rc, "combine_weighted")
    return out


def combine_weighted_bwd(prep: Prepared, g: np.ndarray, rows: np.ndarray | None,
                         w: np.ndarray, init: np.ndarray | None = None, dtype: str = "bf16",
                         fill_pads: bool = True, zero_tail: bool = False):
    """(grad_rows [cap,H] with rows past the live total (unless zero_tail),
    and pad rows when fill_pads is False, left at ``init``; grad_w float64
    [cap] or None; sum of |terms| float64 [cap] or None)."""
    g = _rows(g, dtype)
    T, H = g.shape
    w = np.ascontiguousarray(w, dtype=np.float32)
    st = DTYPES[dtype][1]
    grad_rows = (np.zeros((prep.cap, H), st) if init is None
                 else np.array(init, dtype=st, copy=True))
    gw = aw = None
    if rows is not None:
        rows = _rows(rows, dtype)
        gw = np.zeros(prep.cap, np.float64)
        aw = np.zeros(prep.cap, np.float64)
    rc = _load().ep_oracle_combine_weighted_bwd(T, prep.K, H, DTYPES[dtype][0], int(fill_pads),
                                                int(zero_tail), prep.cap, prep.total,
                                                _p(prep.row_src), _p(g), _p(rows), _p(w),
                                                _p(grad_rows), _p(gw), _p(aw))
    _check(rc, "combine_weighted_bwd")
    return grad_rows, gw, aw
