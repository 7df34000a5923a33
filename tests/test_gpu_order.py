"""GPU: the tile orders and WAVE workgroup sizes give identical results.

The order in which workgroups take the job's tiles (row-major, or XCD-banded:
blocks of 8 rows, a band of columns per XCD) and the size of a WAVE workgroup
(one wave or four) only decide which workgroup computes which (row, group)
unit; the arithmetic of a unit is the same.  So every forced variant must give
the default launch's bits, the default must meet the parity bar against the
oracle, and no variant may write outside the [rows, width] view (the out rows
are padded and guarded).  The shapes cover full and short 8-row blocks, a
partial last tile per row, every kernel family that can take the banded
order, packed groups and both operators.
"""
import numpy as np
import pytest
import torch

import synthetic as S
from gpu_util import (BF16, DT_IDS, F16, F32, FLAG_NBG, FLAG_PER_GROUP, FLAG_RI, assert_parity,
                      dev_buf, host_bits, random_case, say)

pytestmark = pytest.mark.gpu

ROWS, BANDED, WAVE1, WAVE4 = 32, 64, 128, 256


@pytest.fixture(scope="module")
def g():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_group_rmsnorm_amd as g  # raises if libggrms.so is missing

    return g


@pytest.fixture(scope="module")
def orc():
    import oracle

    oracle.build(force=False)
    return oracle


# (dtype, G, groups per row, rows, operator flags)
CASES = [
    (BF16, 128, 60, 37, FLAG_RI),     # WAVE 16 lanes: 15 tiles per row, 4 full 8-row blocks + 5
    (BF16, 128, 7, 9, FLAG_RI),       # 2 tiles per row, the second 3/4 full
    (BF16, 128, 60, 13, FLAG_RI, 4),  # 8-byte vectors (rows padded): 4-wave workgroups
    (BF16, 128, 60, 11, FLAG_RI, 2),  # 4-byte vectors
    (BF16, 8, 100, 19, FLAG_RI),      # WAVE 1 lane: 64 groups per wave, second tile 36/64 full
    (BF16, 512, 9, 17, FLAG_RI),      # WAVE 64 x 1
    (BF16, 576, 13, 11, FLAG_RI),     # WAVE 64 x 2
    (BF16, 768, 10, 19, FLAG_RI),     # BLOCK 128 x 1, one row per workgroup
    (BF16, 896, 9, 33, FLAG_RI),      # BLOCK 128 x 1, 4 rows per workgroup: 9 row tiles
    (BF16, 832, 9, 33, FLAG_RI),      # BLOCK 128 x 1, 2 rows per workgroup: 17 row tiles
    (BF16, 1280, 6, 20, FLAG_RI),     # BLOCK 128 x 2, 4 rows per workgroup
    (BF16, 1088, 6, 20, FLAG_RI),     # BLOCK 128 x 2, 2 rows per workgroup
    (BF16, 4096, 3, 8, FLAG_RI),      # BLOCK 256 x 2, one full block
    (F32, 64, 20, 10, 0),             # f32, 16 lanes
    (F16, 128, 60, 12, FLAG_NBG),     # norm first, per-column weight
    (F16, 100, 48, 300, FLAG_RI),     # packed groups (200 bytes): 16 lanes x 1, one-wave workgroups
    (F16, 100, 48, 1100, FLAG_RI),    # packed groups, a larger job (16 lanes x 1)
    (BF16, 99, 48, 1500, FLAG_RI),    # packed groups in 2-byte pieces, a large job: 16 x 1
                                      # with boundary vectors merged inside each wave
    (BF16, 127, 48, 1500, FLAG_RI),   # half-full 32-lane segments, a large job: runs of 8
    (BF16, 128, 60, 21, FLAG_RI | FLAG_PER_GROUP),  # shared weight: row-major by default
]
VARIANTS = [ROWS, ROWS | WAVE4, ROWS | WAVE1, BANDED, BANDED | WAVE1, BANDED | WAVE4, WAVE1, WAVE4]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{DT_IDS[c[0]]}-G{c[1]}x{c[2]}-r{c[3]}-f{c[4]}"
                         + (f"-pad{c[5]}" if len(c) > 5 else ""))
def test_tile_orders_agree_bitwise(g, orc, case):
    dtype, G, groups, rows, op = case[:5]
    width = G * groups
    sin = width + (case[5] if len(case) > 5 else 0)  # y/gate row stride: padding narrows the vectors
    esz = 4 if dtype == F32 else 2
    pad = 16 // esz
    so = width + pad
    guard = 64
    y, gt, w = random_case(rows, sin, dtype, seed=G + 7 * groups + rows)
    if op & FLAG_PER_GROUP:
        w = np.ascontiguousarray(w[:G])
    yd, gd, wd = dev_buf(y, dtype), dev_buf(gt, dtype), torch.from_numpy(w).cuda()
    canary = {F32: np.float32(-1234.5), F16: np.uint16(0x7BFF), BF16: np.uint16(0x4B4B)}[dtype]
    ob = np.full(guard + (rows - 1) * so + width + guard, canary, dtype=S.storage_dtype(dtype))
    view = np.zeros(ob.shape, dtype=bool)
    for r in range(rows):
        view[guard + r * so: guard + r * so + width] = True
    sp = torch.cuda.current_stream().cuda_stream
    outs = {}
    for extra in [0] + VARIANTS:
        flags = op | extra
        od = dev_buf(ob, dtype)
        # (WAVE_ONE / WAVE_FOUR do nothing for BLOCK launches; nothing here is refused)
        st, p = g.ggrms_plan_tuned(yd.data_ptr(), gd.data_ptr(), wd.data_ptr(), od[guard:].data_ptr(),
                                rows, width, G, sin, sin, so, 1e-5, dtype, flags)
        assert st == g.SUCCESS, f"flags={flags}: {g.ggrms_status_string(st)}"
        say(f"case order {DT_IDS[dtype]} G={G} groups={groups} rows={rows} flags={flags} "
            f"kernel={p['kernel_name']} lanes={p['lanes_per_group']} block={p['block_threads']} "
            f"order={p['tile_order']} workgroups={p['workgroups']}")
        st = g.ggrms_forward_tuned(yd.data_ptr(), gd.data_ptr(), wd.data_ptr(), od[guard:].data_ptr(),
                                rows, width, G, sin, sin, so, 1e-5, dtype, flags, sp)
        assert st == g.SUCCESS, g.ggrms_status_string(st)
        torch.cuda.synchronize()
        got = host_bits(od, dtype)
        assert np.array_equal(got[~view].view(np.uint8), ob[~view].view(np.uint8)), \
            f"flags={flags}: wrote outside the view"
        outs[extra] = (got, p["tile_order"], p["block_threads"])
    ref = orc.forward(y, gt, w, rows=rows, width=width, group_size=G, y_row_stride=sin,
                      gate_row_stride=sin, out_row_stride=so, eps=1e-5, dtype=dtype,
                      round_intermediate=op & FLAG_RI, norm_before_gate=bool(op & FLAG_NBG),
                      weight_per_group=bool(op & FLAG_PER_GROUP), out=ob.copy(), out_offset=guard)
    base = outs[0][0]
    assert_parity(base[view], ref[view], dtype, f"default order, case {case}")
    for extra, (got, order, block) in outs.items():
        assert np.array_equal(got.view(np.uint8), base.view(np.uint8)), \
            f"flags {extra} (order {order}, block {block}) differ from the default launch"
    # the variants did reach both orders
    assert {o for _, o, _ in outs.values()} == {0, 1}
