"""Randomised GPU parity over shapes: top-k from 1 to 64 (every token-group
size of the reduce), experts 1 to 400, alignments 1 to 128, ragged hidden
sizes (short rows, long rows, and rows around the copies' 8 KiB prefetch
rule),
routings around the one-block prepare's cutover, masked, repeated and out-of-range ids, tight and overflowing
capacities, every payload type and both pad policies. Each case runs every
op through the C ABI against the oracle, bit for bit (the weighted backward's
weight gradient within its summation bound), with canaries in every output.
The cases are drawn from a fixed seed, so the set is the same on every run,
and each runs twice: without and with the tail policy (rows past the live
total zeroed).
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
from test_gpu_dtypes import run_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build()


def _cases(n=24):
    rng = np.random.default_rng(20261202)
    out = []
    for i in range(n):
        K = int(rng.choice([1, 2, 3, 5, 7, 8, 9, 13, 16, 21, 32, 33, 63, 64]))
        E = int(rng.integers(1, 301))
        A = int(rng.choice([1, 2, 7, 16, 64]))
        H = int(8 * rng.integers(1, 200))
        T = int(rng.integers(0, 400))
        dt = str(rng.choice(["bf16", "fp16", "fp32"]))
        fill = bool(rng.random() < 0.7)
        kind = str(rng.choice(["distinct", "repeats", "masked", "bad"]))
        cap_kind = str(rng.choice(["worst", "worst", "tight", "zero"]))
        out.append((i, T, K, E, A, H, dt, fill, kind, cap_kind))
    return out


@pytest.mark.parametrize("i,T,K,E,A,H,dt,fill,kind,cap_kind", _cases(),
                         ids=lambda v: str(v) if not isinstance(v, str) else v)
def test_random_shape(i, T, K, E, A, H, dt, fill, kind, cap_kind, zero_tail=False):
    rng = np.random.default_rng(zlib.crc32(f"random-shape-{i}".encode()))
    if kind == "distinct":
        idx = np.argsort(rng.random((T, max(E, K))), axis=1)[:, :K] if T else \
            np.zeros((0, K), np.int64)
        idx = np.where(idx < E, idx, -1)
    elif kind == "repeats":
        idx = rng.integers(0, E, size=(T, K))
    elif kind == "masked":
        idx = np.where(rng.random((T, K)) < 0.85, -1, rng.integers(0, E, size=(T, K)))
    else:
        idx = rng.integers(-3, E + 3, size=(T, K))
    idx = np.asarray(idx, np.int64).reshape(T, K)
    worst = T * K + E * (A - 1)
    cap = {"worst": worst, "tight": worst // 2, "zero": 0}[cap_kind]
    run_case(f"random{i}", idx, E, A, H, cap, dt, fill, rng, zero_tail=zero_tail)


def _long_row_cases(n=8):
    # rows of 8 to 19 KiB: the copies stream the token rows ahead (K >= 4)
    rng = np.random.default_rng(20261203)
    out = []
    for i in range(n):
        K = int(rng.choice([1, 2, 5, 8, 13, 16]))
        E = int(rng.integers(1, 65))
        A = int(rng.choice([1, 4, 16]))
        H = int(8 * rng.integers(513, 1201))
        T = int(rng.integers(0, 201))
        dt = str(rng.choice(["bf16", "fp16", "fp32"]))
        fill = bool(rng.random() < 0.7)
        kind = str(rng.choice(["distinct", "repeats", "masked", "bad"]))
        cap_kind = str(rng.choice(["worst", "worst", "tight"]))
        out.append((100 + i, T, K, E, A, H, dt, fill, kind, cap_kind))
    return out


@pytest.mark.parametrize("i,T,K,E,A,H,dt,fill,kind,cap_kind", _long_row_cases(),
                         ids=lambda v: str(v) if not isinstance(v, str) else v)
def test_random_long_rows(i, T, K, E, A, H, dt, fill, kind, cap_kind):
    test_random_shape(i, T, K, E, A, H, dt, fill, kind, cap_kind)


def _boundary_cases(n=12):
    # routings around the one-block prepare's 4096-route cutover, and rows
    # around the copies' 8 KiB prefetch rule
    rng = np.random.default_rng(20261204)
    out = []
    for i in range(n):
        K = int(rng.choice([1, 2, 3, 8, 9, 16, 64]))
        E = int(rng.integers(1, 400))
        A = int(rng.choice([1, 3, 16, 128]))
        if i % 2 == 0:
            T = max(0, (4096 + int(rng.integers(-200, 200))) // K)
            H = int(8 * rng.integers(1, 40))
        else:
            H = int(8 * rng.choice([255, 256, 257, 511, 512, 513, 1023, 1024, 1025]))
            T = int(rng.integers(0, 200))
        dt = str(rng.choice(["bf16", "fp16", "fp32"]))
        fill = bool(rng.random() < 0.6)
        kind = str(rng.choice(["distinct", "repeats", "masked", "bad"]))
        cap_kind = str(rng.choice(["worst", "worst", "tight"]))
        out.append((200 + i, T, K, E, A, H, dt, fill, kind, cap_kind))
    return out


@pytest.mark.parametrize("i,T,K,E,A,H,dt,fill,kind,cap_kind", _boundary_cases(),
                         ids=lambda v: str(v) if not isinstance(v, str) else v)
def test_random_boundaries(i, T, K, E, A, H, dt, fill, kind, cap_kind):
    test_random_shape(i, T, K, E, A, H, dt, fill, kind, cap_kind)


@pytest.mark.parametrize("i,T,K,E,A,H,dt,fill,kind,cap_kind",
                         _cases() + _long_row_cases() + _boundary_cases(),
                         ids=lambda v: str(v) if not isinstance(v, str) else v)
def test_random_zero_tail(i, T, K, E, A, H, dt, fill, kind, cap_kind):
    """Every random case again under the tail policy: the rows past the live
    total of every expert-major output are zeros, the rest unchanged."""
    test_random_shape(i, T, K, E, A, H, dt, fill, kind, cap_kind, zero_tail=True)


def _medium_cases(n=10):
    # thousands of tokens and rows of 1-16 KiB: several chunks per run list,
    # chunks of 1, 2 and 4 units, the token-row streaming blocks on (K >= 4,
    # rows of 8 KiB or more) and off, and the reduce's token groups at every
    # density
    rng = np.random.default_rng(20261205)
    out = []
    for i in range(n):
        K = int(rng.choice([2, 4, 6, 8]))
        E = int(rng.choice([8, 32, 64, 128, 256]))
        A = int(rng.choice([1, 16, 128]))
        H = int(rng.choice([512, 2048, 4096, 5120, 7168, 8192]))
        T = int(rng.integers(1000, 6001))
        dt = str(rng.choice(["bf16", "fp16", "fp32"]))
        fill = bool(rng.random() < 0.7)
        kind = str(rng.choice(["distinct", "distinct", "masked", "repeats"]))
        cap_kind = str(rng.choice(["worst", "worst", "tight"]))
        out.append((300 + i, T, K, E, A, H, dt, fill, kind, cap_kind))
    return out


@pytest.mark.parametrize("i,T,K,E,A,H,dt,fill,kind,cap_kind", _medium_cases(),
                         ids=lambda v: str(v) if not isinstance(v, str) else v)
def test_random_medium_shapes(i, T, K, E, A, H, dt, fill, kind, cap_kind):
    test_random_shape(i, T, K, E, A, H, dt, fill, kind, cap_kind, zero_tail=bool(i % 2))
