"""Host side of libggrms_example.so (the epilogue called from a producer
kernel): its argument checks, which refuse before any launch, so they run
without a GPU."""
import ctypes
import os

import pytest

PKG = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "gated_group_rmsnorm_amd")


@pytest.fixture(scope="module")
def ex():
    path = os.path.join(PKG, "libggrms_example.so")
    if not os.path.exists(path):
        pytest.fail("libggrms_example.so is not built (python __graft_entry__.py)")
    f = ctypes.CDLL(path).ggrms_example_gemm_norm
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 4 + [ctypes.c_float, ctypes.c_int,
                                                                  ctypes.c_int, ctypes.c_void_p]
    return f


def test_producer_rejects_what_it_does_not_handle(ex):
    """Each call breaks one limit and returns 1 before any HIP call."""
    p = ctypes.c_void_p(1 << 20)  # 16-byte aligned; never dereferenced (every call is refused)
    ok = dict(rows=32, width=1024, K=32, G=512)

    def call(**kw):
        a = dict(ok, **kw)
        return ex(p, p, p, p, p, a["rows"], a["width"], a["K"], a["G"], 1e-5, 1, 0, None)

    assert call(rows=24) == 1             # rows not a multiple of 16
    assert call(rows=0) == 1
    assert call(K=40) == 1                # K not a multiple of 16
    assert call(K=80) == 1                # K above 64
    assert call(G=96, width=960) == 1     # group not a multiple of 64
    assert call(G=2048, width=2048) == 1  # wider than 1024
    assert call(width=1000) == 1          # width not a multiple of the group
    assert ex(None, p, p, p, p, 32, 1024, 32, 512, 1e-5, 1, 0, None) == 1
    q = ctypes.c_void_p((1 << 20) + 8)    # 8-byte aligned only
    assert ex(p, p, q, p, p, 32, 1024, 32, 512, 1e-5, 1, 0, None) == 1
