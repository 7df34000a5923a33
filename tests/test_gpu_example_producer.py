"""The per-unit epilogue called from a producer kernel (libggrms_example.so):
y = bf16(x @ wt^T) computed on the matrix cores and normalised in the same
kernel, against the CPU oracle run on the y that the product defines.

The producer's inputs are small integers times powers of two (x in
{-4..4}/4, wt in {-4..4}/8), so every product and partial sum is exact in
f32 whatever the order of accumulation, and y -- the exact sum rounded once
to bf16 -- is known on the host without the GPU.  Bar: the oracle's 2-ulp
parity on the fused output; y itself (the producer alone) bit for bit; and
the fused output equal bit for bit to the library's WAVE launch of 64 lanes
x 2 vectors on the same y, whose lanes the example's epilogue lays out the
same way."""
import ctypes
import os

import numpy as np
import pytest
import torch

import synthetic as S
from gpu_util import BF16, F32, FLAG_RI, assert_parity, dev_buf, host_bits, run_gpu, say

pytestmark = pytest.mark.gpu

PKG = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "gated_group_rmsnorm_amd")


@pytest.fixture(scope="module")
def g():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_group_rmsnorm_amd as g

    return g


@pytest.fixture(scope="module")
def ex():
    lib = ctypes.CDLL(os.path.join(PKG, "libggrms_example.so"))
    f = lib.ggrms_example_gemm_norm
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 4 + [ctypes.c_float, ctypes.c_int,
                                                                  ctypes.c_int, ctypes.c_void_p]
    return f


@pytest.fixture(scope="module")
def orc():
    import oracle

    oracle.build(force=False)
    return oracle


def small_ints(seed, tid, n):
    """Seeded integers in -4..4 (uniform draws rounded to the nearest)."""
    return np.rint(S.tensor(seed, tid, n, F32, ("uniform", -4.49, 4.49))).astype(np.int64)


CASES = [  # rows, width, K, group size, round_intermediate
    (64, 256, 32, 64, 1),
    (64, 1024, 16, 512, 0),
    (48, 2048, 64, 1024, 1),
    (128, 7680, 64, 960, 1),
    (32, 1920, 48, 960, 0),
    (16, 512, 64, 128, 1),
    (272, 1024, 64, 256, 1),
    # enough tiles that each workgroup takes several in turn (tiles x groups
    # / 256 compute units, at most 16): pairs, an odd count with a single last
    # tile, K below the MFMA's 64, and 16 tiles of 64-wide groups (4 column
    # tiles for 16 waves, 8 live lanes per row)
    (2048, 4096, 64, 512, 1),     # 4 tiles per workgroup
    (4112, 2048, 64, 1024, 0),    # 3 per workgroup, the last one 2
    (8192, 1920, 32, 960, 1),     # 4, K = 32
    (4096, 1024, 16, 64, 1),      # 16, K = 16
]


@pytest.mark.parametrize("rows,width,K,G,ri", CASES)
def test_producer_epilogue_against_the_oracle(g, ex, orc, rows, width, K, G, ri):
    say(f"case example producer rows={rows} width={width} K={K} G={G} ri={ri}")
    seed = 7000 + rows + width + K + G
    xi = small_ints(seed, 11, rows * K).reshape(rows, K)
    wi = small_ints(seed, 12, width * K).reshape(width, K)
    x = S.to_storage((xi / 4.0).astype(np.float32).reshape(-1), BF16)
    wt = S.to_storage((wi / 8.0).astype(np.float32).reshape(-1), BF16)
    # y = x @ wt^T exactly (|sum| <= 16 K / 32), rounded once to bf16
    y32 = ((xi @ wi.T).astype(np.float64) / 32.0).astype(np.float32)
    y = S.to_storage(y32.reshape(-1), BF16)
    gt = S.tensor(seed, S.TID_GATE, rows * width, BF16, ("normal", 1.0))
    w = S.tensor(seed, S.TID_W, width, F32, ("uniform", 0.5, 1.5))
    xd, wtd, gd = dev_buf(x, BF16), dev_buf(wt, BF16), dev_buf(gt, BF16)
    wd = torch.from_numpy(w).cuda()
    s = torch.cuda.current_stream().cuda_stream

    # the producer alone: y bit for bit
    yd = torch.empty(rows * width, dtype=torch.bfloat16, device="cuda")
    assert ex(xd.data_ptr(), wtd.data_ptr(), gd.data_ptr(), wd.data_ptr(), yd.data_ptr(), rows,
              width, K, G, 1e-5, ri, 1, s) == 0
    # fused: y normalised in the producer's epilogue
    od = torch.empty(rows * width, dtype=torch.bfloat16, device="cuda")
    assert ex(xd.data_ptr(), wtd.data_ptr(), gd.data_ptr(), wd.data_ptr(), od.data_ptr(), rows,
              width, K, G, 1e-5, ri, 0, s) == 0
    # the library on the same y, lanes laid out as the example's epilogue
    y_host_d = dev_buf(y, BF16)
    ld = torch.empty_like(od)
    st = run_gpu(g, y_host_d, gd, wd, ld, rows, width, G, width, width, width, 1e-5, BF16, ri,
                 shape=(64, 2), flags=FLAG_RI if ri else 0)
    assert st == g.SUCCESS, g.ggrms_status_string(st)
    torch.cuda.synchronize()

    assert np.array_equal(host_bits(yd, BF16), y), "producer: y differs from the exact product"
    got = host_bits(od, BF16)
    ref = orc.forward(y, gt, w, rows=rows, width=width, group_size=G, y_row_stride=width,
                      gate_row_stride=width, out_row_stride=width, eps=1e-5, dtype=BF16,
                      round_intermediate=ri)
    assert_parity(got, ref, BF16, f"example producer G={G} ri={ri}")
    assert np.array_equal(got, host_bits(ld, BF16)), "fused epilogue differs from the library launch"
