"""GPU: the benchmark's reference stream kernels move the bytes they claim.

The plain two-read-one-write kernels in libggrms_bench.so are what the fused
kernel's times are compared against, so they are checked here like any other
kernel: c = a ^ b over exactly the views given, and nothing outside them
written.  The strided form is checked on the strided small batch's layout
(y and gate as column slices of one [rows, 9856] fp16 buffer, out
contiguous) and on a padded out view.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def aux():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_group_rmsnorm_amd  # noqa: F401  (libggrms.so, which the helpers link)

    lib = ctypes.CDLL(os.path.join(ROOT, "gated_group_rmsnorm_amd", "libggrms_bench.so"))
    lib.ggrms_bench_stream3.restype = ctypes.c_int
    lib.ggrms_bench_stream3.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64, ctypes.c_void_p]
    lib.ggrms_bench_stream3_rows.restype = ctypes.c_int
    lib.ggrms_bench_stream3_rows.argtypes = ([ctypes.c_void_p] * 3 + [ctypes.c_int64] * 5
                                             + [ctypes.c_void_p])
    return lib


def _rand_words(n, seed):
    rng = np.random.default_rng(seed)
    return torch.from_numpy(rng.integers(-2**31, 2**31 - 1, size=n, dtype=np.int64)
                            .astype(np.int32)).cuda()


@pytest.mark.parametrize("rows,width,ld,out_ld", [(256, 4800, 9856, 4800), (7, 4800, 9856, 4808),
                                                  (1, 4800, 4800, 4800), (3, 8, 16, 8),
                                                  (5, 600, 1000, 600)])
def test_stream3_rows_reads_and_writes_the_views(aux, rows, width, ld, out_ld):
    """fp16 views: a = F[:, :width], b = F[:, width:2 width] of F [rows, ld];
    c [rows, width] in a buffer of row stride out_ld filled with a sentinel."""
    print(f"stream3_rows rows={rows} width={width} ld={ld} out_ld={out_ld}", flush=True)
    assert ld >= width
    words = (rows * ld + width) // 2 + 8
    buf = _rand_words(words, rows * 131 + width)
    f16 = buf.view(torch.int16)
    out = torch.full((rows * out_ld,), 0x5A5A, dtype=torch.int16, device="cuda")
    a = f16[:rows * ld].view(rows, ld)[:, :width]
    b = f16[width:width + rows * ld].view(rows, ld)[:, :width]
    rc = aux.ggrms_bench_stream3_rows(a.data_ptr(), b.data_ptr(), out.data_ptr(), rows, width * 2,
                                      ld * 2, ld * 2, out_ld * 2,
                                      torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    got = out.view(rows, out_ld).cpu()
    want = (a.cpu() ^ b.cpu())
    assert torch.equal(got[:, :width], want)
    if out_ld > width:
        assert bool((got[:, width:] == 0x5A5A).all())


def test_stream3_rows_refuses_bad_views(aux):
    """Misaligned strides, a stride below the row, and an empty job are refused
    before any launch."""
    buf = torch.zeros(1024, dtype=torch.int32, device="cuda")
    p = buf.data_ptr()
    s = torch.cuda.current_stream().cuda_stream
    assert aux.ggrms_bench_stream3_rows(p, p, p, 2, 64, 72, 64, 64, s) == 1   # stride % 16
    assert aux.ggrms_bench_stream3_rows(p, p, p, 2, 64, 48, 64, 64, s) == 1   # stride < row
    assert aux.ggrms_bench_stream3_rows(p, p, p, 0, 64, 64, 64, 64, s) == 1   # no rows
    assert aux.ggrms_bench_stream3_rows(p + 8, p, p, 1, 64, 64, 64, 64, s) == 1  # alignment


def test_stream3_flat(aux):
    """The contiguous form: c = a ^ b over nbytes, the bytes after c untouched."""
    n = 4096 + 64
    a, b = _rand_words(n, 1), _rand_words(n, 2)
    c = torch.full((n + 64,), 0x12345678, dtype=torch.int32, device="cuda")
    assert aux.ggrms_bench_stream3(a.data_ptr(), b.data_ptr(), c.data_ptr(), n * 4,
                                   torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    cc = c.cpu()
    assert torch.equal(cc[:n], (a ^ b).cpu())
    assert bool((cc[n:] == 0x12345678).all())
