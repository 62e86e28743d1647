"""Host-side checks of the memory-pattern ceiling library (no GPU needed).

- it loads and exports its entry points (five patterns and the cache flush);
- every size it does not take is refused with 2 before any HIP call (each
  case fails validation, so the fake device addresses are never used);
- the benchmark's pattern sizes fit the buffers it allocates.
"""
import ctypes as C

import pytest

import bench

NAMES = ("epc_write_linear", "epc_write_rows", "epc_read_linear", "epc_copy_linear",
         "epc_gather_sum", "epc_flush")
P = C.c_void_p(0x10000)
P2 = C.c_void_p(0x20000)
S = C.c_void_p(0)


def test_library_exports_its_entry_points():
    lib = bench._ceilings_lib()
    for n in NAMES:
        assert hasattr(lib, n)


def test_sizes_it_does_not_take_are_refused():
    lib = bench._ceilings_lib()
    assert lib.epc_write_linear(None, 1024, S) == 2
    assert lib.epc_write_linear(P, 1000, S) == 2
    assert lib.epc_write_rows(P, 3, 1024, S) == 2          # not a power of two
    assert lib.epc_write_rows(P, 0, 1024, S) == 2
    assert lib.epc_write_rows(P, 4, 1000, S) == 2          # not whole vectors
    assert lib.epc_read_linear(P, 1024, None, S) == 2
    assert lib.epc_read_linear(P, 1025, P2, S) == 2
    assert lib.epc_copy_linear(P, None, 1024, S) == 2
    assert lib.epc_copy_linear(P, P2, 1000, S) == 2
    for k in (0, 3, 5, 6, 7, 9):
        assert lib.epc_gather_sum(P, 16, 1024, 4, k, P2, S) == 2
    assert lib.epc_gather_sum(P, 0, 1024, 4, 2, P2, S) == 2
    assert lib.epc_gather_sum(P, 16, 1000, 4, 2, P2, S) == 2
    assert lib.epc_gather_sum(None, 16, 1024, 4, 2, P2, S) == 2
    assert lib.epc_flush(None, P2, 1024, P, S) == 2
    assert lib.epc_flush(P, None, 1024, P, S) == 2
    assert lib.epc_flush(P, P2, 1024, None, S) == 2
    assert lib.epc_flush(P, P2, 1000, P, S) == 2


@pytest.mark.parametrize("T,K,H", [(4096, 8, 7168), (32768, 8, 7168), (8192, 8, 2048),
                                   (16384, 2, 4096), (256, 2, 512), (100, 3, 520)])
def test_pattern_sizes_fit_the_buffers(T, K, H):
    budget = bench.CEILING_BUFFER_BYTES
    sz = bench.ceiling_sizes(T, K, H)
    row = 2 * H
    n = sz["write_rows"]
    assert n & (n - 1) == 0 and n * row <= budget < 2 * n * row
    assert sz["write_rows_bytes"] == n * row
    g = sz["gather"]
    if K in (1, 2, 4, 8) and T * K * row <= budget:
        assert g == {"ntok": T, "k": K, "nrows": T * K, "row_bytes": row,
                     "bytes": T * K * row + T * row}
        assert g["ntok"] * row <= budget           # the output buffer
    else:
        assert g is None
