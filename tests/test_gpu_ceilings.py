"""The memory-pattern ceiling kernels move the bytes they are timed for.

Each pattern is run once on a small buffer and its effect checked on the
host: the dense and scrambled-row writes zero every byte (the scramble is a
bijection on rows), the copy reproduces its source, and the gather-sum
equals the wrapping 32-bit sum of the hashed rows, including a ragged last
column block.
"""
import numpy as np
import pytest
import torch

import bench

pytestmark = pytest.mark.gpu

SCRAMBLE = 2654435761


def _lib_and_stream():
    torch.cuda.set_device(0)
    return bench._ceilings_lib(), torch.cuda.current_stream().cuda_stream


def test_write_linear_and_copy():
    lib, sp = _lib_and_stream()
    n = 3 << 20
    a = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")
    assert lib.epc_write_linear(a.data_ptr(), n, sp) == 0
    torch.cuda.synchronize()
    assert int(a.count_nonzero()) == 0
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros(n, dtype=torch.uint8, device="cuda")
    assert lib.epc_copy_linear(src.data_ptr(), dst.data_ptr(), n, sp) == 0
    sink = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    assert lib.epc_read_linear(dst.data_ptr(), n, sink.data_ptr(), sp) == 0
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


@pytest.mark.parametrize("nrows,row_bytes", [(64, 14336), (32, 4096), (16, 1040)])
def test_write_rows_covers_every_row(nrows, row_bytes):
    lib, sp = _lib_and_stream()
    a = torch.full((nrows * row_bytes + 4096,), 0xFF, dtype=torch.uint8, device="cuda")
    assert lib.epc_write_rows(a.data_ptr(), nrows, row_bytes, sp) == 0
    torch.cuda.synchronize()
    assert int(a[: nrows * row_bytes].count_nonzero()) == 0
    assert bool((a[nrows * row_bytes:] == 0xFF).all())        # nothing past the rows


@pytest.mark.parametrize("k", [1, 2, 4, 8])
def test_gather_sum_matches_the_hashed_rows(k):
    lib, sp = _lib_and_stream()
    ntok, nrows, row_bytes = 24, 100, 1040                     # 65 vectors: a ragged block
    g = np.random.default_rng(k)
    rows = g.integers(0, 2**32, size=(nrows, row_bytes // 4), dtype=np.uint64).astype(np.uint32)
    d_rows = torch.from_numpy(rows.view(np.int32)).cuda()
    out = torch.full((ntok, row_bytes // 4), -1, dtype=torch.int32, device="cuda")
    assert lib.epc_gather_sum(d_rows.data_ptr(), nrows, row_bytes, ntok, k, out.data_ptr(),
                              sp) == 0
    torch.cuda.synchronize()
    want = np.zeros((ntok, row_bytes // 4), np.uint64)
    for t in range(ntok):
        for j in range(k):
            r = ((t * k + j) * SCRAMBLE) % (1 << 64) % nrows
            want[t] += rows[r]
    want = (want % (1 << 32)).astype(np.uint32)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), want)
