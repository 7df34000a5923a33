"""GPU parity of the ROWS kernel (workgroups that take rows of one group in
turn, the next rows' inputs in flight while they store) against the CPU
oracle, and its bits against the BLOCK kernel with the same lanes and vectors.

Bar as in test_gpu_parity.py: f32 within a relative 1e-5 of the oracle,
fp16/bf16 within 2 units in the last place.  Sizes: forced ROWS launches on
a few hundred rows (every workgroup's loop, its trailing single row and the
prefetch past the last row), and the library's own choice on jobs of 2048+
(row, group) units.
"""
import numpy as np
import pytest
import torch

import synthetic as S
from gpu_util import (BF16, DT_IDS, F16, F32, FLAG_KEEP, FLAG_NBG, FLAG_PER_GROUP, FLAG_RI,
                      FLAG_STREAM, assert_parity, check_contiguous, dev_buf, host_bits,
                      random_case, run_gpu, say)

pytestmark = pytest.mark.gpu

KERNEL_ROWS = 5


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


def _plan(g, rows, width, G, dtype, flags, shape=None):
    n = rows * width * (4 if dtype == F32 else 2)
    st, p = g.ggrms_plan_tuned(1 << 40, (1 << 40) + 2 * n, (1 << 40) + 4 * n, (1 << 40) + 6 * n,
                               rows, width, G, width, width, width, 1e-5, dtype, flags, shape)
    assert st == g.SUCCESS, g.ggrms_status_string(st)
    return p


# (rows, groups per row, G, dtype, lanes x vectors): every built pair, rows
# below, at and above 256 / groups (one row per workgroup; two or three rows
# for some workgroups and one for the rest, so both the paired loop and its
# trailing single row run), several groups per row
FORCED = [
    (300, 1, 4104, BF16, (256, 3)),   # 513 vectors: one past the BLOCK 256 x 2 limit
    (300, 1, 5120, BF16, (320, 2)),
    (37, 1, 5120, BF16, (320, 2)),    # fewer rows than compute units
    (200, 3, 5120, BF16, (320, 2)),   # 85 workgroups per group, 2-3 rows each
    (530, 1, 6144, F16, (384, 2)),
    (260, 2, 7168, BF16, (448, 2)),
    (513, 1, 8192, F16, (512, 2)),
    (300, 1, 2560, F32, (320, 2)),
    (300, 1, 4096, F32, (512, 2)),
    (300, 1, 960, BF16, (256, 3)),    # a narrow group on the widest lanes: most lanes idle
    (300, 1, 12288, BF16, (768, 2)),  # 1536 vectors
    (37, 1, 9216, F16, (768, 2)),     # 1152 vectors, fewer rows than compute units
    (300, 1, 10248, BF16, (768, 2)),  # 1281 vectors: the second slot mostly idle
    (260, 2, 16384, BF16, (1024, 2)), # 2048 vectors, 128 workgroups per group
    (300, 1, 8192, F32, (1024, 2)),
]


@pytest.mark.parametrize("rows,groups,G,dtype,shape", FORCED,
                         ids=[f"{r}x{n}xG{G}-{DT_IDS[d]}-{s[0]}x{s[1]}" for r, n, G, d, s in FORCED])
def test_forced_rows_against_the_oracle(g, orc, rows, groups, G, dtype, shape):
    width = G * groups
    sh = (shape[0], shape[1], 0, 0, KERNEL_ROWS)
    assert _plan(g, rows, width, G, dtype, FLAG_RI, sh)["kernel_name"] == "rows"
    variants = [FLAG_RI, 0, FLAG_NBG, FLAG_RI | FLAG_PER_GROUP] if dtype != F32 else \
        [0, FLAG_NBG, FLAG_PER_GROUP]
    for i, flags in enumerate(variants):
        check_contiguous(g, orc, rows, width, G, dtype, flags & FLAG_RI, seed=9100 + i + rows,
                         shape=sh, flags=flags, tag=f"rows {shape} flags={flags}")


# the library's own choice on jobs large enough for ROWS
AUTO = [(2048, 1, 5120, BF16, 320), (1024, 2, 4864, BF16, 256), (2100, 1, 8192, BF16, 512),
        (2048, 1, 2560, F32, 320), (700, 3, 6152, F16, 448), (2048, 1, 12288, BF16, 768),
        (1100, 2, 14336, F16, 1024)]


@pytest.mark.parametrize("rows,groups,G,dtype,lanes", AUTO,
                         ids=[f"{r}x{n}xG{G}-{DT_IDS[d]}" for r, n, G, d, _ in AUTO])
def test_rows_by_default(g, orc, rows, groups, G, dtype, lanes):
    width = G * groups
    ri = 1 if dtype != F32 else 0
    p = _plan(g, rows, width, G, dtype, FLAG_RI if ri else 0)
    assert (p["kernel_name"], p["lanes_per_group"]) == ("rows", lanes), p
    check_contiguous(g, orc, rows, width, G, dtype, ri, seed=9200 + rows, tag="rows default")


@pytest.mark.parametrize("lanes,vpt,G,dtype", [(256, 3, 5120, BF16), (512, 2, 8192, F16),
                                               (256, 3, 3072, F32), (1024, 2, 16384, BF16)],
                         ids=["256x3-bf16", "512x2-f16", "256x3-f32", "1024x2-bf16"])
def test_rows_equals_block_bitwise(g, lanes, vpt, G, dtype):
    """Same lanes and vectors: the same slots and the same order of the sums,
    so ROWS and BLOCK (one row per workgroup) give the same bits; so do the
    streaming and the cached accesses."""
    rows = 300
    say(f"case rows vs block {lanes}x{vpt} G={G} dtype={DT_IDS[dtype]}")
    y, gt, w = random_case(rows, G, dtype, seed=9300 + G)
    yd, gd, wd = dev_buf(y, dtype), dev_buf(gt, dtype), torch.from_numpy(w).cuda()
    outs = []
    ri = FLAG_RI if dtype != F32 else 0
    for shape, extra in (((lanes, vpt, 1, 0, 0), 0), ((lanes, vpt, 0, 0, KERNEL_ROWS), 0),
                         ((lanes, vpt, 0, 0, KERNEL_ROWS), FLAG_STREAM),
                         ((lanes, vpt, 0, 0, KERNEL_ROWS), FLAG_KEEP)):
        od = torch.empty_like(yd)
        st = run_gpu(g, yd, gd, wd, od, rows, G, G, G, G, G, 1e-5, dtype, 0, shape=shape,
                     flags=ri | extra)
        assert st == g.SUCCESS, g.ggrms_status_string(st)
        outs.append(od)
    torch.cuda.synchronize()
    view = torch.int32 if dtype == F32 else torch.int16
    for o in outs[1:]:
        assert torch.equal(outs[0].view(view), o.view(view))


def test_rows_strided_in_place_and_guarded(g, orc):
    """y and gate as column slices of one fused buffer (16-byte aligned row
    stride), out written in place over y; a second run into a guarded,
    padded out whose padding and guard bands must stay untouched."""
    rows, G, groups = 2304, 5120, 1
    width = G * groups
    fused = 2 * width + 64
    say(f"case rows strided rows={rows} width={width}")
    buf = S.tensor(9401, S.TID_Y, rows * fused, BF16, ("normal", 1.0))
    w = S.tensor(9401, S.TID_W, width, F32, ("uniform", 0.5, 1.5))
    y = buf.reshape(rows, fused)[:, :width]
    gt = buf.reshape(rows, fused)[:, width:2 * width]
    ref = orc.forward(np.ascontiguousarray(y).reshape(-1), np.ascontiguousarray(gt).reshape(-1), w,
                      rows=rows, width=width, group_size=G, y_row_stride=width,
                      gate_row_stride=width, out_row_stride=width, eps=1e-5, dtype=BF16,
                      round_intermediate=1)
    fd, wd = dev_buf(buf, BF16), torch.from_numpy(w).cuda()
    p = g.ggrms_plan_ex(fd.data_ptr(), fd[width:].data_ptr(), wd.data_ptr(), fd.data_ptr(), rows,
                        width, G, fused, fused, fused, 1e-5, BF16, FLAG_RI)[1]
    assert p["kernel_name"] == "rows"
    # into a padded, guarded out
    so, guard = width + 24, 256
    canary = np.uint16(0x4B4B)
    ob = np.full(guard + (rows - 1) * so + width + guard, canary, dtype=np.uint16)
    od = dev_buf(ob, BF16)
    assert run_gpu(g, fd, fd[width:], wd, od[guard:], rows, width, G, fused, fused, so, 1e-5, BF16,
                   1) == g.SUCCESS
    # in place over y
    assert run_gpu(g, fd, fd[width:], wd, fd, rows, width, G, fused, fused, fused, 1e-5, BF16,
                   1) == g.SUCCESS
    torch.cuda.synchronize()
    got = host_bits(od, BF16)
    view = np.zeros(got.shape, dtype=bool)
    for r in range(rows):
        view[guard + r * so:guard + r * so + width] = True
    assert np.array_equal(got[~view], ob[~view])
    assert_parity(got[view], ref, BF16, "rows strided into padded out")
    inplace = host_bits(fd, BF16).reshape(rows, fused)
    assert_parity(np.ascontiguousarray(inplace[:, :width]).reshape(-1), ref, BF16, "rows in place")
    # gate and the padding columns of the fused buffer are untouched
    assert np.array_equal(inplace[:, width:], buf.reshape(rows, fused)[:, width:])


@pytest.mark.parametrize("dtype", [BF16, F16, F32], ids=DT_IDS.get)
def test_rows_special_values(g, orc, dtype):
    """NaN and inf inputs, all-zero groups, gates deep in silu's underflow
    range (the exact path, taken by a whole wave) and large positive gates,
    through a forced ROWS launch whose workgroups take several rows each, in
    both operators."""
    import refs

    G = 5120 if dtype != F32 else 2560
    rows, width = 300, G
    rng = np.random.default_rng(19)
    yv = rng.standard_normal((rows, width))
    gv = rng.standard_normal((rows, width))
    yv[0, 5] = np.nan
    yv[257, 200] = np.inf                          # the second row of a workgroup
    gv[2, 300] = np.nan
    yv[3, :] = 0.0                                 # an all-zero group
    gv[4, :] = rng.uniform(-104, -86, width)       # silu underflow window
    gv[260, :] = -95.0
    gv[6, :] = rng.uniform(80, 100, width)         # silu(x) = x
    gv[7, 7] = -np.inf
    gv[7, 300] = np.inf
    y = refs.round64(yv, dtype).reshape(-1)
    gt = refs.round64(gv, dtype).reshape(-1)
    w = rng.uniform(0.5, 1.5, width).astype(np.float32)
    yd, gd, wd = dev_buf(y, dtype), dev_buf(gt, dtype), torch.from_numpy(w).cuda()
    sh = (320, 2, 0, 0, KERNEL_ROWS)
    for eps in (1e-5, 0.0):
        for flags in ([0, FLAG_RI, FLAG_NBG] if dtype != F32 else [0, FLAG_NBG]):
            say(f"case rows special dtype={DT_IDS[dtype]} eps={eps} flags={flags}")
            od = torch.empty_like(yd)
            assert run_gpu(g, yd, gd, wd, od, rows, width, G, width, width, width, eps, dtype, 0,
                           shape=sh, flags=flags) == g.SUCCESS
            torch.cuda.synchronize()
            ref = orc.forward(y, gt, w, rows=rows, width=width, group_size=G, y_row_stride=width,
                              gate_row_stride=width, out_row_stride=width, eps=eps, dtype=dtype,
                              round_intermediate=flags & FLAG_RI,
                              norm_before_gate=bool(flags & FLAG_NBG))
            assert_parity(host_bits(od, dtype), ref, dtype, f"rows special eps={eps} flags={flags}")


def _draw_rows_case(i: int) -> dict:
    """A seeded random forced-ROWS configuration: a group of 16-byte vectors
    that some built lanes x vectors pair covers, 1-3 groups per row, rows
    around one and two workgroups' worth, 16-byte aligned strided views, both
    operators and both cache policies."""
    rng = np.random.default_rng(20261203 + 104729 * i)
    dtype = int(rng.choice([F32, F16, BF16]))
    per_vec = 4 if dtype == F32 else 8
    nvec = int(rng.integers(1, 1025))
    pairs = [(256, 3), (320, 2), (384, 2), (448, 2), (512, 2)]
    lanes, vpt = pairs[int(rng.integers(0, len(pairs)))]
    nvec = min(nvec, lanes * vpt)
    groups = int(rng.integers(1, 4))
    rows = int(rng.choice([int(rng.integers(1, 40)), int(rng.integers(200, 600))]))
    nbg = bool(rng.random() < 0.3)
    ri = 0 if (nbg or dtype == F32) else int(rng.random() < 0.7)
    per_group = bool(groups > 1 and rng.random() < 0.3)
    flags = ((FLAG_RI if ri else 0) | (FLAG_NBG if nbg else 0) |
             (FLAG_PER_GROUP if per_group else 0) | int(rng.choice([0, FLAG_STREAM, FLAG_KEEP])))
    pad = [int(v) * per_vec for v in rng.integers(0, 3, 3)]  # row strides stay 16-byte multiples
    return dict(dtype=dtype, G=nvec * per_vec, groups=groups, rows=rows, flags=flags, ri=ri,
                shape=(lanes, vpt, 0, 0, KERNEL_ROWS), pads=pad,
                eps=float(rng.choice([1e-5, 1e-6, 0.1])))


N_ROWS_CASES = 24


@pytest.mark.parametrize("i", range(N_ROWS_CASES))
def test_rows_random_forced(g, orc, i):
    c = _draw_rows_case(i)
    dtype, G, rows = c["dtype"], c["G"], c["rows"]
    width = G * c["groups"]
    sy, sg, so = (width + p for p in c["pads"])
    say(f"case rows random {i}: dtype={DT_IDS[dtype]} G={G}x{c['groups']} rows={rows} "
        f"flags={c['flags']} shape={c['shape']} strides={(sy, sg, so)}")
    n_y, n_g, n_o = ((rows - 1) * s + width for s in (sy, sg, so))
    seed = 9500 + i
    y = S.tensor(seed, S.TID_Y, n_y, dtype, ("normal", 1.0))
    gt = S.tensor(seed, S.TID_GATE, n_g, dtype, ("normal", 2.0))
    w = S.tensor(seed, S.TID_W, width, F32, ("uniform", 0.5, 1.5))
    if c["flags"] & FLAG_PER_GROUP:
        w = np.ascontiguousarray(w[:G])
    canary = {F32: np.float32(-1234.5), F16: np.uint16(0x7BFF), BF16: np.uint16(0x4B4B)}[dtype]
    ob = np.full(n_o, canary, dtype=S.storage_dtype(dtype))
    yd, gd, od = dev_buf(y, dtype), dev_buf(gt, dtype), dev_buf(ob, dtype)
    wd = torch.from_numpy(w).cuda()
    st = run_gpu(g, yd, gd, wd, od, rows, width, G, sy, sg, so, c["eps"], dtype, c["ri"],
                 shape=c["shape"], flags=c["flags"])
    assert st == g.SUCCESS, g.ggrms_status_string(st)
    torch.cuda.synchronize()
    got = host_bits(od, dtype)
    ref = ob.copy()
    orc.forward(y, gt, w, rows=rows, width=width, group_size=G, y_row_stride=sy,
                gate_row_stride=sg, out_row_stride=so, eps=c["eps"], dtype=dtype,
                round_intermediate=c["ri"], norm_before_gate=bool(c["flags"] & FLAG_NBG),
                weight_per_group=bool(c["flags"] & FLAG_PER_GROUP), out=ref)
    view = np.zeros(n_o, dtype=bool)
    for r in range(rows):
        view[r * so:r * so + width] = True
    bits = np.uint32 if dtype == F32 else np.uint16
    assert np.array_equal(got[~view].view(bits), ob[~view].view(bits)), "padding written"
    assert_parity(got[view], ref[view], dtype, f"rows random {i}")
