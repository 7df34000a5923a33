"""GPU: seeded random configurations through the C ABI against the oracle.

Each case draws, from its own seed, a dtype, a group size (narrow groups for
the one-wave kernel, medium and wide ones for the multi-wave kernel, and
groups past the register shapes for the two-pass kernel), a number of groups
and rows, the operator (gate first with or without the intermediate cast,
norm first), a per-column or shared weight, the cache policy, the tile order
and WAVE workgroup size, base offsets and padded row strides (which narrow
the vector width down to single elements), a weight pointer off its 16-byte
alignment, in-place output into y or the gate, eps and the input scales.
The library chooses the kernel shape as it does for any caller.  Every case
must meet the parity bar against the oracle inside the [rows, width] view and
leave every other element of the output buffer -- guard bands, padding
columns, and in place the rest of the input buffer -- exactly as it was.

f32 cases keep G <= 4096: above that the f32 oracle's own rounding error can
exceed the 1e-5 bar, and test_group_size_sweep holds those sizes to the exact
result instead.
"""
import numpy as np
import pytest
import torch

import synthetic as S
from gpu_util import (BF16, DT_IDS, F16, F32, FLAG_KEEP, FLAG_NBG, FLAG_PER_GROUP, FLAG_RI,
                      FLAG_STREAM, assert_parity, dev_buf, host_bits, say)

pytestmark = pytest.mark.gpu

ORDER_ROWS, ORDER_BANDED, WAVE_ONE, WAVE_FOUR = 32, 64, 128, 256
N_CASES = 256
GUARD = 64
CANARY = {F32: np.float32(-1234.5), F16: np.uint16(0x7BFF), BF16: np.uint16(0x4B4B)}


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


def draw(i: int) -> dict:
    rng = np.random.default_rng(20261202 + 7919 * i)
    dtype = int(rng.choice([F32, F16, BF16]))
    kind = rng.choice(["narrow", "medium", "wide"], p=[0.5, 0.35, 0.15])
    if kind == "narrow":
        G = int(rng.integers(1, 129))
    elif kind == "medium":
        G = int(rng.integers(129, 1537))
    else:
        G = int(rng.integers(1537, 4097 if dtype == F32 else 9001))
    if rng.random() < 0.5:  # a whole number of 16-byte vectors (for 16-bit data)
        G = max(8, G - G % 8)
    groups = int(rng.integers(1, 4 if kind == "wide" else 9))
    rows = int(rng.integers(1, 7 if kind == "wide" else 41))
    nbg = bool(rng.random() < 0.3)
    ri = 0 if (nbg or dtype == F32) else int(rng.random() < 0.7)
    per_group = bool(groups > 1 and rng.random() < 0.25)
    flags = ((FLAG_RI if ri else 0) | (FLAG_NBG if nbg else 0) |
             (FLAG_PER_GROUP if per_group else 0) |
             int(rng.choice([0, FLAG_STREAM, FLAG_KEEP])) |
             int(rng.choice([0, ORDER_ROWS, ORDER_BANDED])) |
             int(rng.choice([0, WAVE_ONE, WAVE_FOUR])))
    aligned = bool(rng.random() < 0.5)
    offs = (0, 0, 0) if aligned else tuple(int(v) for v in rng.integers(0, 8, 3))
    pads = (0, 0, 0) if aligned else tuple(int(v) for v in rng.integers(0, 9, 3))
    inplace = rng.choice(["none", "y", "gate"], p=[0.85, 0.1, 0.05])
    return dict(i=i, dtype=dtype, G=G, groups=groups, rows=rows, flags=flags, ri=ri, nbg=nbg,
                per_group=per_group, offs=offs, pads=pads, inplace=str(inplace),
                w_off=0 if aligned else int(rng.integers(0, 4)),
                eps=float(rng.choice([1e-5, 1e-6, 0.1])),
                y_scale=float(rng.choice([0.5, 1.0, 4.0])),
                gate_scale=float(rng.choice([1.0, 2.0, 4.0])))


def _case_id(i):
    c = draw(i)
    return f"{i}-{DT_IDS[c['dtype']]}-G{c['G']}x{c['groups']}-r{c['rows']}-f{c['flags']}-{c['inplace']}"


@pytest.mark.parametrize("i", range(N_CASES), ids=_case_id)
def test_random_configuration(g, orc, i):
    c = draw(i)
    dtype, G, rows = c["dtype"], c["G"], c["rows"]
    width = G * c["groups"]
    oy, og, oo = c["offs"]
    sy, sg, so = width + c["pads"][0], width + c["pads"][1], width + c["pads"][2]
    if c["inplace"] != "none":  # out is exactly y or the gate: same pointer and stride
        oo, so = (oy, sy) if c["inplace"] == "y" else (og, sg)
    say(f"case random {_case_id(i)} offs={(oy, og, oo)} strides={(sy, sg, so)} "
        f"w_off={c['w_off']} eps={c['eps']}")
    n_y = oy + (rows - 1) * sy + width
    n_g = og + (rows - 1) * sg + width
    seed = 5000 + i
    yb = S.tensor(seed, S.TID_Y, n_y, dtype, ("normal", c["y_scale"]))
    gb = S.tensor(seed, S.TID_GATE, n_g, dtype, ("normal", c["gate_scale"]))
    wlen = G if c["per_group"] else width
    w = S.tensor(seed, S.TID_W, wlen, F32, ("uniform", 0.5, 1.5))

    yd, gd = dev_buf(yb, dtype), dev_buf(gb, dtype)
    wbuf = torch.zeros(wlen + 4, dtype=torch.float32, device="cuda")
    wbuf[c["w_off"]:c["w_off"] + wlen] = torch.from_numpy(w).cuda()
    if c["inplace"] == "y":
        od, base, before, o_at = yd, 0, yb, oo
    elif c["inplace"] == "gate":
        od, base, before, o_at = gd, 0, gb, oo
    else:
        n_o = oo + (rows - 1) * so + width
        before = np.full(GUARD + n_o + GUARD, CANARY[dtype], dtype=S.storage_dtype(dtype))
        od, base, o_at = dev_buf(before, dtype), GUARD, GUARD + oo
    y_ptr = yd[oy:].data_ptr()
    g_ptr = gd[og:].data_ptr()
    o_ptr = od[base + oo:].data_ptr()
    w_ptr = wbuf[c["w_off"]:].data_ptr()
    st = g.ggrms_forward_tuned(y_ptr, g_ptr, w_ptr, o_ptr, rows, width, G, sy, sg, so, c["eps"],
                            dtype, c["flags"], torch.cuda.current_stream().cuda_stream)
    assert st == g.SUCCESS, g.ggrms_status_string(st)
    torch.cuda.synchronize()
    got = host_bits(od, dtype)

    ref = before.copy()
    orc.forward(yb, gb, w, rows=rows, width=width, group_size=G, y_row_stride=sy,
                gate_row_stride=sg, out_row_stride=so, eps=c["eps"], dtype=dtype,
                round_intermediate=c["ri"], norm_before_gate=c["nbg"],
                weight_per_group=c["per_group"], out=ref, y_offset=oy, gate_offset=og,
                out_offset=o_at)
    view = np.zeros(ref.shape, dtype=bool)
    for r in range(rows):
        view[o_at + r * so:o_at + r * so + width] = True
    bits = np.uint32 if dtype == F32 else np.uint16
    outside = ~view
    assert np.array_equal(got[outside].view(bits), before[outside].view(bits)), \
        f"case {i}: elements outside the view changed"
    assert_parity(got[view], ref[view], dtype, f"random case {_case_id(i)}")


N_PACKED_CASES = 96
KERNEL_RUN = 4


def draw_packed(i: int) -> dict:
    """A packed layout: 16-byte aligned rows whose groups are not a whole number
    of 16-byte vectors (more than one vector each), in runs of groups or on
    lane segments, with a per-column weight or one shared by every group."""
    rng = np.random.default_rng(77003 + 104729 * i)
    dtype = int(rng.choice([F32, F16, BF16]))
    esz = 4 if dtype == F32 else 2
    while True:
        G = int(rng.integers(17 // esz + 1, 700 if dtype != F32 else 300))
        if (G * esz) % 16:
            break
    pb = int(np.gcd(G * esz, 16))
    period = 16 // pb  # groups that make a 16-byte aligned row
    kmax = max(1, min(96 // period, 16384 // (G * period)))  # rows of at most 16384 elements
    groups = period * int(rng.integers(1, kmax + 1))
    rows = int(rng.choice([1, 2, 3, 7, 33, 130, 600]))
    nbg = bool(rng.random() < 0.3)
    ri = 0 if (nbg or dtype == F32) else int(rng.random() < 0.7)
    per_group = bool(groups > 1 and rng.random() < 0.3)
    shape = ["default", "run", "run1", "run2", "wave"][int(rng.integers(0, 5))]
    flags = ((FLAG_RI if ri else 0) | (FLAG_NBG if nbg else 0) |
             (FLAG_PER_GROUP if per_group else 0) |
             int(rng.choice([0, ORDER_ROWS, ORDER_BANDED])) | int(rng.choice([0, WAVE_FOUR])))
    pad16 = 16 // esz  # a row stride padded by whole 16-byte vectors keeps rows aligned
    pads = tuple(int(v) * pad16 for v in rng.integers(0, 3, 3))
    offs = tuple(int(v) * pad16 for v in rng.integers(0, 3, 3))
    inplace = str(rng.choice(["none", "gate"], p=[0.85, 0.15]))
    return dict(i=i, dtype=dtype, G=G, groups=groups, rows=rows, flags=flags, ri=ri, nbg=nbg,
                per_group=per_group, shape=shape, pads=pads, offs=offs, inplace=inplace,
                eps=float(rng.choice([1e-5, 1e-6])))


def _packed_id(i):
    c = draw_packed(i)
    return (f"{i}-{DT_IDS[c['dtype']]}-G{c['G']}x{c['groups']}-r{c['rows']}-f{c['flags']}-"
            f"{c['shape']}-{c['inplace']}")


@pytest.mark.parametrize("i", range(N_PACKED_CASES), ids=_packed_id)
def test_random_packed_configuration(g, orc, i):
    """Packed groups under seeded random launch choices (the library's, runs
    with its or a forced vector count, lane segments with boundaries merged)
    against the oracle, guard bands and padding untouched; the plan must be
    packed, and the forced kernel family the one that runs."""
    c = draw_packed(i)
    dtype, G, rows = c["dtype"], c["G"], c["rows"]
    esz = 4 if dtype == F32 else 2
    width = G * c["groups"]
    oy, og, oo = c["offs"]
    sy, sg, so = width + c["pads"][0], width + c["pads"][1], width + c["pads"][2]
    if c["inplace"] == "gate":
        oo, so = og, sg
    n_y = oy + (rows - 1) * sy + width
    n_g = og + (rows - 1) * sg + width
    seed = 9000 + i
    yb = S.tensor(seed, S.TID_Y, n_y, dtype, ("normal", 1.0))
    gb = S.tensor(seed, S.TID_GATE, n_g, dtype, ("normal", 2.0))
    wlen = G if c["per_group"] else width
    w = S.tensor(seed, S.TID_W, wlen, F32, ("uniform", 0.5, 1.5))
    yd, gd = dev_buf(yb, dtype), dev_buf(gb, dtype)
    wd = torch.from_numpy(w).cuda()
    if c["inplace"] == "gate":
        od, base, before, o_at = gd, 0, gb, oo
    else:
        n_o = oo + (rows - 1) * so + width
        before = np.full(GUARD + n_o + GUARD, CANARY[dtype], dtype=S.storage_dtype(dtype))
        od, base, o_at = dev_buf(before, dtype), GUARD, GUARD + oo
    ptrs = (yd[oy:].data_ptr(), gd[og:].data_ptr(), wd.data_ptr(), od[base + oo:].data_ptr())
    shape = {"default": None, "run": (0, 0, 0, 0, KERNEL_RUN), "run1": (64, 1, 0, 0, KERNEL_RUN),
             "run2": (64, 2, 0, 0, KERNEL_RUN), "wave": None}[c["shape"]]
    st, p = g.ggrms_plan_tuned(*ptrs, rows, width, G, sy, sg, so, c["eps"], dtype, c["flags"])
    assert st == g.SUCCESS, g.ggrms_status_string(st)
    assert p["vector_bytes"] == 16 and p["piece_bytes"] < 16, p
    if c["shape"] == "wave" and p["lanes_per_group"] <= 64:
        lanes = 1
        while lanes < p["lanes_per_group"] * p["vectors_per_lane"]:
            lanes *= 2
        shape = (lanes, 1)
    if shape is not None:
        st2, p2 = g.ggrms_plan_tuned(*ptrs, rows, width, G, sy, sg, so, c["eps"], dtype,
                                     c["flags"], shape)
        if st2 != g.SUCCESS:  # a run that two groups do not fit, a segment past 64 lanes
            assert st2 == g.ERROR_NOT_SUPPORTED, g.ggrms_status_string(st2)
            shape, p2 = None, p
        p = p2
    say(f"case random packed {_packed_id(i)} offs={(oy, og, oo)} strides={(sy, sg, so)} "
        f"plan={p['kernel_name']} {p['lanes_per_group']}x{p['vectors_per_lane']} "
        f"runs of {p['groups_per_run']}")
    if shape is not None and len(shape) == 5:
        assert p["kernel_name"] == "run", p
    st = g.ggrms_forward_tuned(*ptrs, rows, width, G, sy, sg, so, c["eps"], dtype, c["flags"],
                               torch.cuda.current_stream().cuda_stream, shape)
    assert st == g.SUCCESS, g.ggrms_status_string(st)
    torch.cuda.synchronize()
    got = host_bits(od, dtype)
    ref = before.copy()
    orc.forward(yb, gb, w, rows=rows, width=width, group_size=G, y_row_stride=sy,
                gate_row_stride=sg, out_row_stride=so, eps=c["eps"], dtype=dtype,
                round_intermediate=c["ri"], norm_before_gate=c["nbg"],
                weight_per_group=c["per_group"], out=ref, y_offset=oy, gate_offset=og,
                out_offset=o_at)
    view = np.zeros(ref.shape, dtype=bool)
    for r in range(rows):
        view[o_at + r * so:o_at + r * so + width] = True
    bits = np.uint32 if dtype == F32 else np.uint16
    assert np.array_equal(got[~view].view(bits), before[~view].view(bits)), \
        f"case {i}: elements outside the view changed"
    assert_parity(got[view], ref[view], dtype, f"random packed case {_packed_id(i)}")
