"""The C ABI on the CPU: the library loads, exports what include/ggrms.h and
include/ggrms_tuning.h declare, rejects bad arguments before any HIP call, and
plans kernels as documented.  Nothing here launches a kernel or needs a GPU."""
import ctypes
import math
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ggrms.h")
TUNING_HEADER = os.path.join(ROOT, "include", "ggrms_tuning.h")
HEADERS = (HEADER, TUNING_HEADER)

F32, F16, BF16 = 0, 1, 2
OK, INVALID, NOTSUP = 0, 1, 2
A = 1 << 20  # a 256-byte aligned fake device address (never dereferenced)


@pytest.fixture(scope="module")
def g():
    import gated_group_rmsnorm_amd as g

    return g


def _declared_functions(headers=HEADERS):
    text = "".join(open(h).read() for h in headers)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ggrms_[a-z_]+)\s*\(", text)))


def test_header_symbols_exported(g):
    names = _declared_functions()
    assert {"ggrms_forward", "ggrms_plan", "ggrms_status_string", "ggrms_abi_version"} <= set(names)
    # the launch controls live in the tuning header only
    assert set(_declared_functions((TUNING_HEADER,))) == {"ggrms_forward_tuned", "ggrms_plan_tuned"}
    assert not {"ggrms_forward_tuned", "ggrms_plan_tuned"} & set(_declared_functions((HEADER,)))
    lib = ctypes.CDLL(g.library_path())
    for n in names:
        assert hasattr(lib, n), f"{n} declared in ggrms.h but not exported"
    # the dynamic symbol table holds the header's functions and nothing else
    # (no internal C++ symbols, no kernel handles)
    out = subprocess.run(["nm", "-D", "--defined-only", g.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if len(l.split()) == 3}
    assert exported == set(names), (f"exported but undeclared: {sorted(exported - set(names))[:5]}; "
                                    f"declared but not exported: {sorted(set(names) - exported)}")
    assert all(l.split()[1] == "T" for l in out.splitlines() if len(l.split()) == 3)


def test_abi_version_and_strings(g):
    assert g.ggrms_abi_version() == 5
    for st in range(4):
        assert g.ggrms_status_string(st)
    assert g.ggrms_status_string(99) == "unknown status"


def _header_constants(headers=HEADERS):
    """NAME -> value of every enumerator and integer #define in the headers."""
    text = re.sub(r"/\*.*?\*/", "", "".join(open(h).read() for h in headers), flags=re.S)
    consts = {n: int(v) for n, v in re.findall(r"\b(GGRMS_[A-Z0-9_]+)\s*=\s*(\d+)\s*[,}\n]", text)}
    for n, v in re.findall(r"#define\s+(GGRMS_[A-Z0-9_]+)\s+(.+)", text):
        m = re.fullmatch(r"\(?(\d+)(?:ll)?(?:\s*<<\s*(\d+))?\)?", v.strip())
        if m:  # an integer literal, possibly shifted
            consts[n] = int(m[1]) << int(m[2] or 0)
    return consts


def test_binding_constants_match_header(g):
    """Every enumerator and integer macro of the headers has the same value in
    the Python binding (named without the GGRMS_ prefix, or, for the kernel
    ids, as keys of KERNEL_NAMES)."""
    consts = _header_constants()
    assert len(consts) >= 22, sorted(consts)
    tuning = _header_constants((TUNING_HEADER,))
    assert {n for n in tuning if n.startswith("GGRMS_FLAG_")} == {
        "GGRMS_FLAG_CACHE_STREAM", "GGRMS_FLAG_CACHE_KEEP", "GGRMS_FLAG_ORDER_ROWS",
        "GGRMS_FLAG_ORDER_BANDED", "GGRMS_FLAG_WAVE_ONE", "GGRMS_FLAG_WAVE_FOUR"}
    for name, value in consts.items():
        short = name[len("GGRMS_"):]
        if short.startswith("KERNEL_"):
            assert g.KERNEL_NAMES[value] == short[len("KERNEL_"):].lower(), name
        elif short == "ABI_VERSION":
            assert g.ABI_VERSION == value == g.ggrms_abi_version()
        else:
            assert getattr(g, short) == value, f"{name} = {value} in the header"
            assert short in g.__all__, short
    assert set(g.KERNEL_NAMES) == {v for n, v in consts.items() if n.startswith("GGRMS_KERNEL_")}


def _fwd(g, **kw):
    args = dict(y=A, gate=A + (1 << 24), norm_weight=A + (2 << 24), out=A + (3 << 24), rows=4,
                width=256, group_size=64, y_row_stride=256, gate_row_stride=256,
                out_row_stride=256, eps=1e-5, dtype=BF16, round_intermediate=1)
    args.update(kw)
    st_plan, plan = g.ggrms_plan(*args.values())
    # ggrms_forward is only called where its checks reject the arguments (or
    # there is nothing to launch), so no call here reaches the HIP runtime.
    st_fwd = g.ggrms_forward(*args.values(), 0) if (st_plan != OK or args["rows"] == 0) else None
    return st_plan, st_fwd, plan


BAD = [
    dict(rows=-1), dict(width=0), dict(group_size=0), dict(group_size=-64), dict(group_size=48),
    dict(y=0), dict(gate=0), dict(norm_weight=0), dict(out=0),
    dict(y_row_stride=255), dict(gate_row_stride=100), dict(out_row_stride=-256),
    dict(y=A + 1), dict(out=A + (3 << 24) + 1), dict(norm_weight=A + (2 << 24) + 2),
    dict(dtype=F32, y=A + 2),
    dict(round_intermediate=2), dict(round_intermediate=-1),
    dict(eps=float("nan")), dict(eps=float("inf")), dict(eps=-1e-5),
    # out overlapping an input other than exactly in place
    dict(out=A + 2), dict(out=A, out_row_stride=512),
    dict(out=A + (1 << 24) + 64),
    # out overlapping the weight (which every row reads): at its start, ending in it,
    # and a strided out whose second row meets it
    dict(out=A + (2 << 24)), dict(out=A + (2 << 24) - 2046),
    dict(out=A + (2 << 24) - 2048 - 256, out_row_stride=1024),
    # extents that overflow 64-bit addressing
    dict(rows=1 << 40, y_row_stride=1 << 40, gate_row_stride=1 << 40, out_row_stride=1 << 40),
]


@pytest.mark.parametrize("kw", BAD, ids=lambda k: ",".join(f"{a}={v}" for a, v in k.items()))
def test_invalid_arguments(g, kw):
    st_plan, st_fwd, _ = _fwd(g, **kw)
    assert st_plan == INVALID and st_fwd == INVALID


def test_unknown_dtype(g):
    st_plan, st_fwd, _ = _fwd(g, dtype=7)
    assert st_plan == NOTSUP and st_fwd == NOTSUP


def test_zero_rows_is_a_no_op(g):
    st_plan, st_fwd, plan = _fwd(g, rows=0, y=0, gate=0, out=0, norm_weight=0)
    assert st_plan == OK and st_fwd == OK and plan["kernel_name"] == "none"


def test_single_row_ignores_strides(g):
    st, plan = g.ggrms_plan(A, A + 4096, A + 8192, A + 12288, 1, 256, 64, 0, 0, 0, 1e-5, BF16, 1)
    assert st == OK and plan["vector_bytes"] == 16


def test_in_place_is_allowed(g):
    for alias in ("y", "gate"):
        kw = {"out": A if alias == "y" else A + (1 << 24)}
        st, _, plan = _fwd(g, **kw)
        assert st == OK, alias


def test_interleaved_views_do_not_overlap(g):
    """y and gate as column slices of one fused buffer, out in a third
    column slice of the same buffer: no element is shared, so it is allowed."""
    st, _, plan = _fwd(g, rows=8, width=100, group_size=100, y=A, gate=A + 200, out=A + 400,
                       y_row_stride=300, gate_row_stride=300, out_row_stride=300, dtype=F16)
    assert st == OK
    st, _, _ = _fwd(g, rows=8, width=100, group_size=100, y=A, gate=A + 200, out=A + 398,
                    y_row_stride=300, gate_row_stride=300, out_row_stride=300, dtype=F16)
    assert st == INVALID


RI, NBG, PER_GROUP, STREAM, KEEP = 1, 2, 4, 8, 16
KERNEL_RUN, KERNEL_ROWS = 4, 5
ROWS, BANDED, WAVE1, WAVE4 = 32, 64, 128, 256


TUNING = STREAM | KEEP | ROWS | BANDED | WAVE1 | WAVE4


def _plan_ex(g, flags, shape=None, **kw):
    """ggrms_plan_tuned (ggrms_plan_ex when no launch control is set: both must
    agree), checking that the forward entry points return the same status
    wherever it rejects the arguments."""
    args = dict(y=A, gate=A + (1 << 24), norm_weight=A + (2 << 24), out=A + (3 << 24), rows=4,
                width=256, group_size=64, y_row_stride=256, gate_row_stride=256,
                out_row_stride=256, eps=1e-5, dtype=BF16)
    args.update(kw)
    st, plan = g.ggrms_plan_tuned(*args.values(), flags, shape)
    if shape is None and not flags & TUNING:
        st_ex, plan_ex = g.ggrms_plan_ex(*args.values(), flags)
        assert (st_ex, plan_ex) == (st, plan)
    if st != OK or args["rows"] == 0:
        # rejected (or nothing to launch): the forward entry point returns
        # the same status without reaching the HIP runtime
        assert g.ggrms_forward_tuned(*args.values(), flags, 0, shape) == st
        if shape is None and not flags & TUNING:
            assert g.ggrms_forward_ex(*args.values(), flags, 0) == st
    return st, plan


def test_weight_in_the_gap_of_a_strided_out(g):
    """A weight (1024 bytes here) that lies between two rows (512 bytes each)
    of a strided out shares no byte with it: allowed; one byte further and
    a row meets it."""
    W = A + (2 << 24)
    # rows 4096 bytes apart: row 0 ends 1536 bytes before the weight, row 1 starts after it
    st_plan, _, _ = _fwd(g, out=W - 2048, out_row_stride=2048, rows=2)
    assert st_plan == OK
    # row 0 ends exactly where the weight starts
    st_plan, _, _ = _fwd(g, out=W - 512, out_row_stride=2048, rows=2)
    assert st_plan == OK
    st_plan, _, _ = _fwd(g, out=W - 510, out_row_stride=2048, rows=2)
    assert st_plan == INVALID
    # row 1 starts exactly where the weight ends, or one element earlier
    st_plan, _, _ = _fwd(g, out=W + 1024 - 4096, out_row_stride=2048, rows=2)
    assert st_plan == OK
    st_plan, _, _ = _fwd(g, out=W + 1022 - 4096, out_row_stride=2048, rows=2)
    assert st_plan == INVALID


@pytest.mark.parametrize("flags", [STREAM, KEEP, ROWS, BANDED, WAVE1, WAVE4, RI | STREAM])
def test_ex_calls_refuse_launch_controls(g, flags):
    """The launch controls belong to the _tuned calls; the _ex calls reject
    them like unknown bits."""
    args = (A, A + (1 << 24), A + (2 << 24), A + (3 << 24), 4, 256, 64, 256, 256, 256, 1e-5, BF16)
    assert g.ggrms_plan_ex(*args, flags)[0] == INVALID
    assert g.ggrms_forward_ex(*args, flags, 0) == INVALID
    assert g.ggrms_plan_tuned(*args, flags)[0] == OK


@pytest.mark.parametrize("flags", [512, 1 << 31, RI | NBG, RI | NBG | PER_GROUP,
                                   STREAM | KEEP, RI | STREAM | KEEP, ROWS | BANDED,
                                   WAVE1 | WAVE4, RI | ROWS | BANDED, RI | WAVE1 | WAVE4])
def test_invalid_flags(g, flags):
    assert _plan_ex(g, flags)[0] == INVALID


@pytest.mark.parametrize("flags", [0, RI, NBG, PER_GROUP, RI | PER_GROUP, NBG | PER_GROUP,
                                   RI | STREAM, NBG | KEEP, PER_GROUP | STREAM])
def test_valid_flags_plan_like_the_default(g, flags):
    """The operator variants and cache policies use the same kernel shapes:
    only the arithmetic, the weight's stride between groups and the cache
    hint differ."""
    st, p = _plan_ex(g, flags, rows=64, width=7680, group_size=960, y_row_stride=7680,
                     gate_row_stride=7680, out_row_stride=7680,
                     gate=A + (1 << 26), norm_weight=A + (2 << 26), out=A + (3 << 26))
    assert st == OK
    st, ref = g.ggrms_plan(A, A + (1 << 26), A + (2 << 26), A + (3 << 26), 64, 7680, 960, 7680,
                           7680, 7680, 1e-5, BF16, 1)
    # 64 rows x 7680 bf16 x 3 views = 2.9 MB: below the streaming threshold
    assert ref["streaming"] == 0
    assert p["streaming"] == (1 if flags & STREAM else 0)
    p.pop("streaming"), ref.pop("streaming")
    assert p == ref


def test_tile_order_and_wave_workgroups(g):
    """WAVE workgroups are one wave for 16-byte vectors and four waves for
    narrower vectors and packed groups; the XCD-banded order is taken when every
    group has its own weights and a row's tiles (one per workgroup) are not a
    multiple of 8; the launch controls force either."""
    kw = dict(gate=A + (1 << 30), norm_weight=A + (2 << 30), out=A + (3 << 30))

    def plan(flags, rows, width, G, dtype=BF16, stride=None, **more):
        st, p = _plan_ex(g, flags, rows=rows, width=width, group_size=G,
                         y_row_stride=stride or width, gate_row_stride=stride or width,
                         out_row_stride=width, dtype=dtype, **{**kw, **more})
        assert st == OK, (flags, rows, width, G)
        return p

    # 60 groups of 128 bf16 per row, 4 per wave: 15 waves per row -> banded, one tile per wave
    p = plan(RI, 8192, 7680, 128)
    assert (p["kernel_name"], p["tile_order"], p["block_threads"], p["workgroups"]) == \
        ("wave", 1, 64, 8192 * 15)
    # the same groups sharing one weight: row-major
    p = plan(RI | PER_GROUP, 8192, 7680, 128)
    assert (p["tile_order"], p["block_threads"], p["workgroups"]) == (0, 64, 8192 * 60 // 4)
    # forced row-major order and 4-wave workgroups: a row-major run of 16 units each
    p = plan(RI | ROWS | WAVE4, 8192, 7680, 128)
    assert (p["tile_order"], p["block_threads"], p["workgroups"]) == (0, 256, 8192 * 60 // 16)
    # forced banded with 4-wave workgroups: tiles of 16 groups, 4 per row (the last 3/4 full)
    p = plan(RI | BANDED | WAVE4, 8192, 7680, 128)
    assert (p["tile_order"], p["block_threads"], p["workgroups"]) == (1, 256, 8192 * 4)
    # a partial last tile per row: 7 groups of 128 -> 2 waves per row, the second 3/4 full
    p = plan(RI, 100, 896, 128)
    assert (p["tile_order"], p["workgroups"]) == (1, 100 * 2)
    # 8-byte vectors (rows padded by 4 bf16): 4-wave workgroups of 8 groups; 60 groups are
    # 7.5 of them, so row-major workgroups would straddle rows -> banded, 8 tiles per row
    # (the last half full)
    p = plan(RI, 1024, 7680, 128, stride=7684)
    assert (p["vector_bytes"], p["block_threads"], p["tile_order"], p["workgroups"]) == \
        (8, 256, 1, 1024 * 8)
    # 64 such groups: exactly 8 workgroups per row -> row-major
    p = plan(RI, 1024, 8192, 128, stride=8196)
    assert (p["vector_bytes"], p["block_threads"], p["tile_order"], p["workgroups"]) == \
        (8, 256, 0, 1024 * 8)
    # 4-byte vectors: 64 lanes per group, 4 groups per workgroup, 15 tiles -> banded
    p = plan(RI, 1024, 7680, 128, stride=7682)
    assert (p["vector_bytes"], p["block_threads"], p["tile_order"], p["workgroups"]) == \
        (4, 256, 1, 1024 * 15)
    # BLOCK, 9 groups of 896 bf16 (4 rows per workgroup): banded over 16 x 9 tiles
    p = plan(RI, 64, 8064, 896)
    assert (p["kernel_name"], p["rows_per_workgroup"], p["tile_order"], p["workgroups"]) == \
        ("block", 4, 1, 16 * 9)
    # 9 groups of 832 (2 rows per workgroup): 32 x 9 tiles
    p = plan(RI, 64, 7488, 832)
    assert (p["kernel_name"], p["rows_per_workgroup"], p["tile_order"], p["workgroups"]) == \
        ("block", 2, 1, 32 * 9)
    # 8 groups of 960: a multiple of 8 tiles per row -> row-major; banded if forced
    assert plan(RI, 8192, 7680, 960)["tile_order"] == 0
    p = plan(RI | BANDED, 8192, 7680, 960)
    assert (p["tile_order"], p["workgroups"]) == (1, 8192 // 4 * 8)
    # WIDE is always row-major
    assert plan(RI | BANDED, 4, 3 * 40960, 40960)["tile_order"] == 0
    # packed groups (200-byte groups of the strided layout, a job of 3072 waves at 16
    # lanes per group, resident at once): 16 lanes x 1 vector per group in one-wave
    # workgroups of 4 groups, 12 per row, banded (800-byte tiles: super-tiles of 4,
    # 3200 bytes, 25 cache lines); four waves if forced (3 tiles of 3200 bytes per
    # row); row-major if forced
    fused = dict(y=A, gate=A + 9600)
    p = plan(RI, 256, 4800, 100, F16, stride=9856, **fused)
    assert (p["lanes_per_group"], p["vectors_per_lane"], p["piece_bytes"], p["block_threads"],
            p["tile_order"], p["super_tile"], p["workgroups"]) == (16, 1, 8, 64, 1, 4, 256 * 12)
    p = plan(RI | WAVE4, 256, 4800, 100, F16, stride=9856, **fused)
    assert (p["block_threads"], p["tile_order"], p["super_tile"], p["workgroups"]) == \
        (256, 1, 1, 256 * 3)
    p = plan(RI | ROWS, 256, 4800, 100, F16, stride=9856, **fused)
    assert (p["block_threads"], p["tile_order"], p["super_tile"], p["workgroups"]) == \
        (64, 0, 1, 256 * 48 * 16 // 64)
    # a larger packed job (12288 waves): 16 lanes x 1 vector per group (8-byte
    # pieces), 800-byte tiles in super-tiles of 4 (3200 bytes, 25 lines)
    p = plan(RI, 1024, 4800, 100, F16, stride=9856, **fused)
    assert (p["kernel_name"], p["lanes_per_group"], p["vectors_per_lane"], p["block_threads"],
            p["workgroups"], p["tile_order"], p["super_tile"]) == ("wave", 16, 1, 64, 1024 * 12, 1, 4)
    # 64 such groups per row: 16 tiles, a multiple of the 8 XCDs, banded all the same
    p = plan(RI, 1024, 6400, 100, F16)
    assert (p["tile_order"], p["super_tile"], p["workgroups"]) == (1, 4, 1024 * 16)
    # 36 per row: 9 tiles, no power of two above 1 divides them -> plain banded
    p = plan(RI, 1024, 3600, 100, F16)
    assert (p["tile_order"], p["super_tile"], p["workgroups"]) == (1, 1, 1024 * 9)
    # 40 per row: 10 tiles -> super-tiles of 2 (1600 bytes, half a line over)
    p = plan(RI, 1024, 4000, 100, F16)
    assert (p["tile_order"], p["super_tile"]) == (1, 2)
    # 99-wide bf16 groups (2-byte pieces, 12.4 vectors on 16 lanes) in a large job: 16 x 1,
    # 792-byte tiles in super-tiles of 4 (16 would be whole lines, but 12 tiles per row)
    p = plan(RI, 1024, 48 * 99, 99, BF16)
    assert (p["kernel_name"], p["lanes_per_group"], p["vectors_per_lane"], p["groups_per_run"],
            p["workgroups"], p["tile_order"], p["super_tile"]) == ("wave", 16, 1, 0, 1024 * 12, 1, 4)
    # 127-wide bf16 groups (15.9 vectors on 32 lanes, half-full segments): runs of 8 groups
    # (2032 bytes, 127 vectors: two per lane, every run on a vector boundary), 6 runs per
    # row, banded in super-tiles of 2 runs (8 would make whole 128-byte lines, 2 divides 6)
    p = plan(RI, 1024, 48 * 127, 127, BF16)
    assert (p["kernel_name"], p["lanes_per_group"], p["vectors_per_lane"], p["groups_per_run"],
            p["block_threads"], p["workgroups"], p["tile_order"], p["super_tile"]) == \
        ("run", 64, 2, 8, 64, 1024 * 6, 1, 2)
    # 40 such groups per row: 5 runs -> banded
    p = plan(RI, 1024, 40 * 127, 127, BF16)
    assert (p["kernel_name"], p["workgroups"], p["tile_order"]) == ("run", 1024 * 5, 1)

    # one row: banded over the row's tiles (XCD x takes a run of columns)
    p = plan(RI, 1, 7680, 128)
    assert (p["tile_order"], p["workgroups"]) == (1, 15)


def test_cache_policy_by_job_size(g):
    """Jobs of at least STREAM_MIN_BYTES (y, gate and out together) stream;
    smaller ones keep their lines cached; the flags override either way."""
    assert g.STREAM_MIN_BYTES == 4 << 20
    # 4 MiB exactly: 3 views x rows x width x 2 B with width 1024 -> rows = 4 MiB / 6 KiB
    # is not an integer; use f32 width 1024 (4 KiB rows, 12 KiB per row over the views):
    # 341 rows = 4,190,208 B (below), 342 rows = 4,202,496 B (at or above)
    kw = dict(width=1024, group_size=1024, y_row_stride=1024, gate_row_stride=1024,
              out_row_stride=1024, dtype=F32, gate=A + (1 << 26), norm_weight=A + (2 << 26),
              out=A + (3 << 26))
    assert _plan_ex(g, 0, rows=341, **kw)[1]["streaming"] == 0
    assert _plan_ex(g, 0, rows=342, **kw)[1]["streaming"] == 1
    assert _plan_ex(g, STREAM, rows=1, **kw)[1]["streaming"] == 1
    assert _plan_ex(g, KEEP, rows=342, **kw)[1]["streaming"] == 0
    # padded row strides do not count: only the [rows, width] views' bytes
    kw.update(y_row_stride=4096, gate_row_stride=4096)
    assert _plan_ex(g, 0, rows=341, **kw)[1]["streaming"] == 0


def test_per_group_weight_extent(g):
    """A per-group weight spans group_size floats, a per-column one width
    floats: a weight that ends 512 bytes below the top of the address space
    holds a 64-value group weight but not a 256-column one."""
    top = (1 << 64) - 512
    assert _plan_ex(g, 0, norm_weight=top)[0] == INVALID
    assert _plan_ex(g, PER_GROUP, norm_weight=top)[0] == OK
    assert _plan_ex(g, NBG | PER_GROUP, norm_weight=top)[0] == OK


def test_plan_ex_with_shape(g):
    st, p = _plan_ex(g, NBG, shape=(64, 2), width=960, group_size=960, y_row_stride=960,
                     gate_row_stride=960, out_row_stride=960)
    assert st == OK and (p["kernel_name"], p["lanes_per_group"], p["vectors_per_lane"]) == ("wave", 64, 2)
    st, p = _plan_ex(g, RI, shape=(128, 1, 2), width=960, group_size=960, y_row_stride=960,
                     gate_row_stride=960, out_row_stride=960)
    assert st == OK and (p["lanes_per_group"], p["rows_per_workgroup"], p["lds_bytes"]) == (128, 2, 3840)
    assert _plan_ex(g, 0, shape=(64, 1), width=960, group_size=960, y_row_stride=960,
                    gate_row_stride=960, out_row_stride=960)[0] == NOTSUP
    # all zero: the library's own choice
    assert _plan_ex(g, 0, shape=(0, 0)) == _plan_ex(g, 0)
    assert _plan_ex(g, 0, shape=(128, 1, -1), width=1024, group_size=1024, y_row_stride=1024,
                    gate_row_stride=1024, out_row_stride=1024)[0] == INVALID
    for bad in ((-1, 1), (64, -1), (64, 1, 0, 3), (64, 1, 0, 32), (64, 1, 0, -16)):
        assert _plan_ex(g, 0, shape=bad)[0] == INVALID, bad


def test_plan_with_vector_bytes(g):
    """A forced vector width: the table's shape for the vectors it gives, or
    the forced lanes and vectors; refused where the alignment or the element
    size does not allow it."""
    kw = dict(rows=1, width=7680, group_size=960, y_row_stride=7680, gate_row_stride=7680,
              out_row_stride=7680, gate=A + (1 << 26), norm_weight=A + (2 << 26),
              out=A + (3 << 26))
    want = {16: ("block", 128, 1), 8: ("block", 256, 1), 4: ("block", 256, 2)}
    for vb, (kern, lanes, vpt) in want.items():
        st, p = _plan_ex(g, RI, shape=(0, 0, 0, vb), **kw)
        assert st == OK and (p["vector_bytes"], p["piece_bytes"]) == (vb, vb), vb
        assert (p["kernel_name"], p["lanes_per_group"], p["vectors_per_lane"]) == (kern, lanes, vpt)
    st, p = _plan_ex(g, RI, shape=(512, 1, 0, 4), **kw)
    assert st == OK and (p["lanes_per_group"], p["workgroups"], p["block_threads"]) == (512, 8, 512)
    # 2-byte vectors of f32 are smaller than an element; 16-byte vectors need 16-byte views
    assert _plan_ex(g, 0, shape=(0, 0, 0, 2), dtype=F32)[0] == NOTSUP
    assert _plan_ex(g, RI, shape=(0, 0, 0, 16), **{**kw, "y": A + 8})[0] == NOTSUP
    # a forced width below 16 never packs: 100 fp16 (200 bytes) in 8-byte vectors
    pk = dict(rows=7, width=1600, group_size=100, y_row_stride=1600, gate_row_stride=1600,
              out_row_stride=1600, dtype=F16, gate=A + (1 << 26), norm_weight=A + (2 << 26),
              out=A + (3 << 26))
    assert _plan_ex(g, RI, **pk)[1]["piece_bytes"] == 8
    st, p = _plan_ex(g, RI, shape=(0, 0, 0, 8), **pk)
    assert st == OK and (p["vector_bytes"], p["piece_bytes"], p["lanes_per_group"]) == (8, 8, 32)
    st, p = _plan_ex(g, RI, shape=(0, 0, 0, 16), **pk)
    assert st == OK and (p["vector_bytes"], p["piece_bytes"]) == (16, 8)


def _plan(g, rows, width, G, dtype, sy=None, sg=None, so=None, y=A, gate=A + (1 << 30),
          w=A + (2 << 30), out=A + (3 << 30)):
    sy = width if sy is None else sy
    sg = width if sg is None else sg
    so = width if so is None else so
    st, p = g.ggrms_plan(y, gate, w, out, rows, width, G, sy, sg, so, 1e-5, dtype, 1)
    assert st == OK
    return p


def test_plans_for_the_workloads(g):
    # 8192x7680 bf16, G = 960: 120 16-byte vectors per group -> two waves, one vector per lane
    # and four rows of one group per workgroup, sharing the group's weights in LDS
    p = _plan(g, 8192, 7680, 960, BF16)
    assert (p["kernel_name"], p["vector_bytes"], p["lanes_per_group"], p["vectors_per_lane"]) == ("block", 16, 128, 1)
    assert (p["rows_per_workgroup"], p["block_threads"], p["lds_bytes"]) == (4, 512, 960 * 4)
    assert p["workgroups"] == 8192 // 4 * 8 and p["launches"] == 1
    # decode 1x7680: 8 groups of two waves, one row per workgroup, no staging
    p = _plan(g, 1, 7680, 960, BF16)
    assert (p["workgroups"], p["rows_per_workgroup"], p["lds_bytes"]) == (8, 1, 0)
    # three rows: two per workgroup
    assert _plan(g, 3, 7680, 960, BF16)["rows_per_workgroup"] == 2
    # weights not 16-byte aligned: no staging
    p = _plan(g, 64, 7680, 960, BF16, w=A + (2 << 30) + 16)
    assert p["rows_per_workgroup"] == 4
    p = _plan(g, 64, 7680, 960, F32, w=A + (2 << 30) + 8)
    assert p["rows_per_workgroup"] == 1
    # 16384x8192 fp16, G = 128: 16 vectors -> 16-lane segments, four groups per wave
    p = _plan(g, 16384, 8192, 128, F16)
    assert (p["kernel_name"], p["vector_bytes"], p["lanes_per_group"], p["vectors_per_lane"]) == ("wave", 16, 16, 1)
    # one wave per workgroup (4 groups each), row-major: a row's 16 waves are a multiple
    # of 8, so every XCD already keeps to two of them (a weight per column); with the head
    # scale shared by every group the order does not matter either
    assert (p["block_threads"], p["workgroups"], p["tile_order"]) == (64, 16384 * 16, 0)
    st, p = _plan_ex(g, PER_GROUP, rows=16384, width=8192, group_size=128, y_row_stride=8192,
                     gate_row_stride=8192, out_row_stride=8192, dtype=F16, gate=A + (1 << 30),
                     norm_weight=A + (2 << 30), out=A + (3 << 30))
    assert st == OK and (p["block_threads"], p["workgroups"], p["tile_order"]) == (64, 16384 * 16, 0)
    # 256x4800 fp16 slices of a [256, 9856] buffer, G = 100: 200-byte groups in 9600-byte
    # rows -> packed: 16-byte vectors from the row start, boundary vectors in 8-byte pieces;
    # a group touches at most ceil((8 + 200) / 16) = 13 vectors -> 16 lanes with one
    # vector each, boundary vectors inside a wave merged
    p = _plan(g, 256, 4800, 100, F16, sy=9856, sg=9856, y=A, gate=A + 9600)
    assert (p["kernel_name"], p["vector_bytes"], p["piece_bytes"], p["lanes_per_group"],
            p["vectors_per_lane"]) == ("wave", 16, 8, 16, 1)
    # one-wave workgroups of 4 groups, 12 per row -> banded
    assert (p["block_threads"], p["workgroups"], p["tile_order"]) == (64, 256 * 12, 1)
    # tiny f32, G = 64: 16 vectors
    p = _plan(g, 4, 256, 64, F32)
    assert (p["vector_bytes"], p["lanes_per_group"]) == (16, 16)
    # cache policy: the prefill (377 MB), GDN-shaped (805 MB) and strided (7.4 MB) jobs
    # stream; decode (77 KB) and the tiny case keep their lines cached
    assert _plan(g, 8192, 7680, 960, BF16)["streaming"] == 1
    assert _plan(g, 16384, 8192, 128, F16)["streaming"] == 1
    assert _plan(g, 256, 4800, 100, F16, sy=9856, sg=9856, y=A, gate=A + 9600)["streaming"] == 1
    assert _plan(g, 1, 7680, 960, BF16)["streaming"] == 0
    assert _plan(g, 4, 256, 64, F32)["streaming"] == 0


@pytest.mark.parametrize("G,dtype,pb,nvec", [
    (100, F16, 8, 13),     # 200-byte groups
    (99, BF16, 2, 14),     # 198 bytes: gcd 2, up to 14 bytes before the first boundary
    (50, BF16, 4, 7),      # 100 bytes
    (9, BF16, 2, 2),       # 18 bytes: just over one vector
    (5, F32, 4, 2),        # 20 bytes
    (1001, F32, 4, 251),
    (8191, F16, 2, 1025),  # BLOCK 512 x 3 (packed groups keep one row per workgroup)
])
def test_packed_groups_plan(g, G, dtype, pb, nvec):
    """Groups whose byte length is not a multiple of 16, in rows that are:
    16-byte vectors, pieces of gcd(group bytes, 16), one row per workgroup,
    a shape covering the worst-aligned group."""
    width = 16 * G
    p = _plan(g, 7, width, G, dtype)
    assert (p["vector_bytes"], p["piece_bytes"], p["rows_per_workgroup"]) == (16, pb, 1)
    assert p["lanes_per_group"] * p["vectors_per_lane"] >= nvec
    assert p["lanes_per_group"] * p["vectors_per_lane"] < 2 * nvec or p["lanes_per_group"] == 1


def test_packed_groups_need_aligned_rows(g):
    """The packed path only when every row is 16-byte aligned and a multiple
    of 16 bytes long, the weight is per column and 16-byte aligned or one
    weight is shared by every group (any 4-byte alignment), and a group is
    more than one vector and at most 2048 vectors; otherwise the widest
    vector the group allows."""
    G = 100
    ok = _plan(g, 7, 16 * G, G, F16)
    assert (ok["vector_bytes"], ok["piece_bytes"]) == (16, 8)
    # rows of 3 groups: 600 bytes, not a multiple of 16
    assert (_plan(g, 7, 3 * G, G, F16)["vector_bytes"], _plan(g, 7, 3 * G, G, F16)["piece_bytes"]) == (8, 8)
    # a base pointer only 8-byte aligned; a row stride that breaks 16-byte rows
    assert _plan(g, 7, 16 * G, G, F16, y=A + 8)["vector_bytes"] == 8
    assert _plan(g, 7, 16 * G, G, F16, sg=16 * G + 4)["vector_bytes"] == 8
    # ... but a single row ignores its strides
    assert _plan(g, 1, 16 * G, G, F16, sg=16 * G + 4)["piece_bytes"] == 8
    # weight only 8-byte aligned: 4-byte vectors (two fp16 values, two 4-byte weights)
    p = _plan(g, 7, 16 * G, G, F16, w=A + (2 << 30) + 8)
    assert (p["vector_bytes"], p["piece_bytes"]) == (4, 4)
    # one weight per group position (shared by every group), read piece by piece: packed
    # when the weight is aligned to a piece's weights (8-byte pieces: 4 floats, 16 bytes;
    # 2-byte pieces of 127 bf16: one float)
    for Gs, dt, woff, packed in ((G, F16, 0, True), (G, F16, 8, False), (127, BF16, 4, True)):
        st, p = _plan_ex(g, PER_GROUP, rows=7, width=16 * Gs, group_size=Gs,
                         y_row_stride=16 * Gs, gate_row_stride=16 * Gs, out_row_stride=16 * Gs,
                         dtype=dt, gate=A + (1 << 26), norm_weight=A + (2 << 26) + woff,
                         out=A + (3 << 26))
        assert st == OK and (p["vector_bytes"] == 16 and p["piece_bytes"] < 16) == packed, \
            (Gs, woff, p)
    # ... and in runs, which stage it in LDS (groups of at most 512 elements)
    st, p = _plan_ex(g, PER_GROUP | RI, rows=30000, width=16 * 127, group_size=127,
                     y_row_stride=16 * 127, gate_row_stride=16 * 127, out_row_stride=16 * 127,
                     dtype=BF16, gate=A + (1 << 28), norm_weight=A + (2 << 28), out=A + (3 << 28))
    assert st == OK and (p["kernel_name"], p["piece_bytes"], p["lds_bytes"]) == ("run", 2, 127 * 4)
    # groups of at most one vector (14 bytes)
    assert _plan(g, 7, 16 * 7, 7, BF16)["vector_bytes"] == 2
    # 16381 bf16 = 32762 bytes: 2049 vectors, above the packed limit
    p = _plan(g, 3, 16 * 16381, 16381, BF16)
    assert (p["vector_bytes"], p["kernel_name"]) == (2, "wide")
    # forced shapes: WIDE and staged rows are not built packed
    st, _ = _plan_ex(g, RI, shape=(1024, 0), rows=7, width=16 * G, group_size=G,
                     y_row_stride=16 * G, gate_row_stride=16 * G, out_row_stride=16 * G, dtype=F16,
                     gate=A + (1 << 26), norm_weight=A + (2 << 26), out=A + (3 << 26))
    assert st == NOTSUP
    st, _ = _plan_ex(g, RI, shape=(16, 1, 2), rows=7, width=16 * G, group_size=G,
                     y_row_stride=16 * G, gate_row_stride=16 * G, out_row_stride=16 * G, dtype=F16,
                     gate=A + (1 << 26), norm_weight=A + (2 << 26), out=A + (3 << 26))
    assert st == NOTSUP
    # a covering shape can be forced; one that does not cover 13 vectors cannot
    st, p = _plan_ex(g, RI, shape=(64, 1), rows=7, width=16 * G, group_size=G,
                     y_row_stride=16 * G, gate_row_stride=16 * G, out_row_stride=16 * G, dtype=F16,
                     gate=A + (1 << 26), norm_weight=A + (2 << 26), out=A + (3 << 26))
    assert st == OK and (p["lanes_per_group"], p["piece_bytes"]) == (64, 8)
    st, _ = _plan_ex(g, RI, shape=(8, 1), rows=7, width=16 * G, group_size=G,
                     y_row_stride=16 * G, gate_row_stride=16 * G, out_row_stride=16 * G, dtype=F16,
                     gate=A + (1 << 26), norm_weight=A + (2 << 26), out=A + (3 << 26))
    assert st == NOTSUP


def test_rows_plan(g):
    """ROWS: groups of 513-1792 16-byte vectors that are not packed, in jobs of
    at least 2048 (row, group) units with at most 256 groups per row: one
    workgroup per compute unit (256 / groups per group, at most one per row),
    256 lanes x 3 up to 608 vectors, two vectors on the next multiple of 64
    lanes up to 1024, 768 x 2 up to 1536 and 1024 x 2 above; one launch, no
    banded order.  Forced through the tuning shape's kernel field for any
    group of at most 2048 16-byte vectors (the library's lanes, or a built
    pair that covers the group); refused for narrower vectors, packed groups,
    unbuilt pairs and several rows per workgroup."""
    kw = dict(gate=A + (1 << 30), norm_weight=A + (2 << 30), out=A + (3 << 30))

    def plan(rows, G, dtype=BF16, groups=1, flags=RI, shape=None, **more):
        width = G * groups
        args = dict(rows=rows, width=width, group_size=G, y_row_stride=width,
                    gate_row_stride=width, out_row_stride=width, dtype=dtype, **kw)
        args.update(more)
        return _plan_ex(g, flags, shape, **args)

    # the rule by vectors per group (bf16: 8 elements per vector; f32: 4)
    for G, dtype, lanes, vpt in ((4104, BF16, 256, 3), (4864, BF16, 256, 3), (4872, BF16, 320, 2),
                                 (5120, BF16, 320, 2), (5128, BF16, 384, 2), (6144, F16, 384, 2),
                                 (6152, BF16, 448, 2), (7168, BF16, 448, 2), (7176, BF16, 512, 2),
                                 (8192, BF16, 512, 2), (2560, F32, 320, 2), (4096, F32, 512, 2),
                                 (8200, BF16, 768, 2), (12288, BF16, 768, 2),
                                 (12296, BF16, 1024, 2), (14336, BF16, 1024, 2),
                                 (7168, F32, 1024, 2)):
        st, p = plan(12288, G, dtype)
        assert st == OK and (p["kernel_name"], p["lanes_per_group"], p["vectors_per_lane"],
                             p["block_threads"], p["workgroups"], p["launches"], p["tile_order"],
                             p["rows_per_workgroup"], p["lds_bytes"]) == \
            ("rows", lanes, vpt, lanes, 256, 1, 0, 48, 0), (G, dtype, p)
        assert plan(12288, G, dtype, shape=(0, 0, 0, 0, KERNEL_ROWS))[1] == p
        assert plan(12288, G, dtype, shape=(lanes, vpt, 1, 16, KERNEL_ROWS))[1] == p
        # norm first and a shared weight: the same choice
        assert plan(12288, G, dtype, flags=NBG)[1]["kernel_name"] == "rows"
        assert plan(12288, G, dtype, flags=RI | PER_GROUP, groups=2)[1]["kernel_name"] == "rows"
    # several groups per row: 256 / groups workgroups per group; at least 2048 units
    st, p = plan(1024, 5120, groups=2)
    assert (p["kernel_name"], p["workgroups"], p["rows_per_workgroup"]) == ("rows", 256, 8)
    st, p = plan(700, 5120, groups=3)
    assert (p["kernel_name"], p["workgroups"], p["rows_per_workgroup"]) == ("rows", 255, 9)
    assert plan(1023, 5120, groups=2)[1]["kernel_name"] == "block"
    assert plan(2047, 5120)[1]["kernel_name"] == "block"
    assert plan(2048, 5120)[1]["kernel_name"] == "rows"
    # wider and narrower groups, narrower vectors, a strided view that is
    # not 16-byte aligned: the other kernels
    assert plan(12288, 14344)[1]["kernel_name"] == "block"
    assert plan(12288, 16384)[1]["kernel_name"] == "block"
    assert plan(12288, 4096)[1]["kernel_name"] == "block"
    # ... but up to 2048 vectors it can be forced
    st, p = plan(12288, 16384, shape=(0, 0, 0, 0, KERNEL_ROWS))
    assert st == OK and (p["kernel_name"], p["lanes_per_group"], p["vectors_per_lane"]) == \
        ("rows", 1024, 2)
    p = plan(12288, 5120, y_row_stride=5124)[1]
    assert (p["kernel_name"], p["vector_bytes"]) == ("block", 8)
    # a forced ROWS launch with fewer rows than compute units: one workgroup per row
    st, p = plan(100, 5120, shape=(0, 0, 0, 0, KERNEL_ROWS))
    assert st == OK and (p["workgroups"], p["rows_per_workgroup"]) == (100, 1)
    st, p = plan(300, 960, shape=(0, 0, 0, 0, KERNEL_ROWS))
    assert st == OK and (p["lanes_per_group"], p["vectors_per_lane"], p["workgroups"],
                         p["rows_per_workgroup"]) == (256, 3, 256, 2)
    st, p = plan(300, 960, shape=(320, 2, 0, 0, KERNEL_ROWS))
    assert st == OK and (p["kernel_name"], p["lanes_per_group"]) == ("rows", 320)
    # refusals: more than 2048 vectors, packed groups, narrower vectors, pairs
    # not built or too small, rows per workgroup
    assert plan(300, 16392, shape=(0, 0, 0, 0, KERNEL_ROWS))[0] == NOTSUP
    assert plan(300, 12296, shape=(768, 2, 0, 0, KERNEL_ROWS))[0] == NOTSUP
    assert plan(300, 12296, shape=(640, 2, 0, 0, KERNEL_ROWS))[0] == NOTSUP
    assert plan(300, 100, dtype=F16, groups=16, shape=(0, 0, 0, 0, KERNEL_ROWS))[0] == NOTSUP
    assert plan(300, 5120, shape=(0, 0, 0, 8, KERNEL_ROWS))[0] == NOTSUP
    assert plan(300, 5120, shape=(256, 4, 0, 0, KERNEL_ROWS))[0] == NOTSUP
    assert plan(300, 5120, shape=(256, 3, 0, 0, KERNEL_ROWS))[0] == OK
    assert plan(300, 6144, shape=(320, 2, 0, 0, KERNEL_ROWS))[0] == NOTSUP
    assert plan(300, 5120, shape=(320, 2, 2, 0, KERNEL_ROWS))[0] == NOTSUP
    assert plan(300, 5120, shape=(0, 0, 0, 0, 6))[0] == INVALID


def test_runs_of_packed_groups_plan(g):
    """Runs: packed groups of at most 32 vectors that fill less than 60% of
    their lane segment, in a job of more than 4096 waves, when the run fills
    at least half of its slots; the run is the one that fills the most of its 64 x (1 or 2) slots,
    a run that spans a whole number of vectors (a multiple of 16 / piece
    bytes groups) counting 0.1 more, two vectors per lane on a tie, at most
    32 groups; one-wave workgroups; forced through the tuning shape's kernel
    field (optionally with the vectors per lane) for any packed group that
    fits twice; refused for groups that are not packed, or
    groups too wide for two per wave; a shared weight only for groups of at
    most 512 elements (staged in LDS)."""
    kw = dict(gate=A + (1 << 30), norm_weight=A + (2 << 30), out=A + (3 << 30))
    def plan(rows, G, dtype, groups=16, flags=RI, shape=None):
        width = G * groups
        return _plan_ex(g, flags, shape, rows=rows, width=width, group_size=G, y_row_stride=width,
                        gate_row_stride=width, out_row_stride=width, dtype=dtype, **kw)

    def run_rule(gb, pb, force=0):  # -> (groups per run, vectors per lane)
        best, pick = -1.0, (0, 0)
        for v in (2, 1):
            if force and v != force:
                continue
            cap = 64 * 16 * v
            ga = min(cap // gb, 32) // (16 // pb) * (16 // pb)
            gm = min((cap - 16 + pb) // gb, 32)
            fa = ga * gb / cap + 0.1 if ga >= 2 else -1.0
            fm = gm * gb / cap if gm >= 2 else -1.0
            cand = (fa, ga) if fa >= fm else (fm, gm)
            if cand[0] > best + 1e-9:
                best, pick = cand[0], (cand[1], v)
        return pick

    cases = ((100, F16), (99, BF16), (50, BF16), (127, BF16), (250, F16), (25, F32), (99, F32),
             (13, F16), (68, F16), (76, F16), (84, F16), (140, BF16), (150, BF16), (180, BF16))
    chosen = {}
    for G, dtype in cases:
        esz = 4 if dtype == F32 else 2
        gb = G * esz
        pb = math.gcd(gb, 16)
        gpw, vpt = run_rule(gb, pb)
        lanes = 1
        while lanes < (16 - pb + gb + 15) // 16:
            lanes *= 2
        default = lanes < 64 and 2 * gpw * gb >= 64 * 16 * vpt and 10 * gb < 6 * 16 * lanes
        st, p = plan(8000, G, dtype, shape=(0, 0, 0, 0, KERNEL_RUN))
        assert st == OK and (p["kernel_name"], p["groups_per_run"], p["vectors_per_lane"],
                             p["block_threads"], p["workgroups"]) == \
            ("run", gpw, vpt, 64, 8000 * (-(-16 // gpw))), (G, dtype, p)
        assert p["lanes_per_group"] == 64
        chosen[(G, dtype)] = (gpw, vpt, default)
        assert plan(8000, G, dtype, shape=(64, vpt, 0, 16, KERNEL_RUN))[1] == p
        for v in (1, 2):  # a forced vector count takes the best run for it
            st, q = plan(8000, G, dtype, shape=(64, v, 0, 0, KERNEL_RUN))
            want = run_rule(gb, pb, v)
            if want[0] >= 2:
                assert st == OK and (q["groups_per_run"], q["vectors_per_lane"]) == want, (G, v, q)
            else:
                assert st == NOTSUP, (G, v)
        assert (plan(8000, G, dtype)[1] == p) == default, (G, dtype)
        # a small job stays on lane segments; a run can be forced
        st, q = plan(20, G, dtype)
        assert q["kernel_name"] == "wave", (G, q)
        st, q = plan(20, G, dtype, shape=(0, 0, 0, 0, KERNEL_RUN))
        assert st == OK and q["kernel_name"] == "run" and q["groups_per_run"] == gpw
    # anchors: aligned runs of 10 100-wide fp16 groups (125 vectors) and of 8 127-wide
    # bf16 groups (127 vectors) on two vectors per lane, 32 13-wide fp16 groups (52
    # vectors) on one; only the last two by default
    assert chosen[(100, F16)] == (10, 2, False)
    assert chosen[(127, BF16)] == (8, 2, True)
    assert chosen[(13, F16)] == (32, 1, True)
    # groups of 33-38 vectors (64-lane segments under 60% full) stay WAVE by default and
    # run three to a wave on two vectors per lane if forced; groups of <= 2 vectors stay WAVE
    assert plan(8000, 300, F16)[1]["kernel_name"] == "wave"
    st, p = plan(8000, 300, F16, shape=(0, 0, 0, 0, KERNEL_RUN))
    assert (p["kernel_name"], p["groups_per_run"], p["vectors_per_lane"]) == ("run", 3, 2)
    assert plan(8000, 9, BF16)[1]["kernel_name"] == "wave"
    # refusals: aligned groups, a shared weight, a group too wide for two in 128 vectors,
    # other lane or vector shapes
    assert plan(2000, 128, F16, shape=(0, 0, 0, 0, KERNEL_RUN))[0] == NOTSUP
    st, p = plan(2000, 100, F16, flags=RI | PER_GROUP, shape=(0, 0, 0, 0, KERNEL_RUN))
    assert st == OK and (p["kernel_name"], p["lds_bytes"]) == ("run", 400)
    assert plan(2000, 516, F16, flags=RI | PER_GROUP, shape=(0, 0, 0, 0, KERNEL_RUN))[0] == NOTSUP
    assert plan(2000, 1100, F16, shape=(0, 0, 0, 0, KERNEL_RUN))[0] == NOTSUP
    assert plan(2000, 300, F16, shape=(64, 1, 0, 0, KERNEL_RUN))[0] == NOTSUP
    assert plan(2000, 100, F16, shape=(32, 1, 0, 0, KERNEL_RUN))[0] == NOTSUP
    assert plan(2000, 100, F16, shape=(64, 3, 0, 0, KERNEL_RUN))[0] == NOTSUP
    assert plan(2000, 100, F16, shape=(64, 1, 2, 0, KERNEL_RUN))[0] == NOTSUP
    assert plan(2000, 100, F16, shape=(0, 0, 0, 0, 7))[0] == INVALID
    # 8 groups per row: one run of all 8 (2032 bytes, two vectors per lane)
    st, p = plan(50000, 127, BF16, groups=8)
    assert (p["kernel_name"], p["groups_per_run"], p["workgroups"]) == ("run", 8, 50000)
    # 24 groups per row: three runs of 8
    st, p = plan(50000, 127, BF16, groups=24)
    assert (p["kernel_name"], p["groups_per_run"], p["workgroups"]) == ("run", 8, 50000 * 3)


def test_rows_split_over_launches(g):
    """A grid that would pass 2^31 threads is split by rows: with 1024
    threads per group (BLOCK 1024 x 1 or WIDE, forced) a launch takes at most
    2^21 groups."""
    rows, G = (1 << 21) + 3, 8
    for shape in ((1024, 1), (1024, 0)):
        st, p = _plan_ex(g, RI, shape=shape, rows=rows, width=G, group_size=G, y_row_stride=G,
                         gate_row_stride=G, out_row_stride=G, gate=A + (1 << 26),
                         norm_weight=A + (2 << 26), out=A + (3 << 26))
        assert st == OK
        assert (p["launches"], p["workgroups"], p["block_threads"]) == (2, rows, 1024), shape
    # two groups per row: 2^20 rows per launch
    st, p = _plan_ex(g, RI, shape=(1024, 1), rows=(1 << 20) + 1, width=2 * G, group_size=G,
                     y_row_stride=2 * G, gate_row_stride=2 * G, out_row_stride=2 * G,
                     gate=A + (1 << 26), norm_weight=A + (2 << 26), out=A + (3 << 26))
    assert st == OK and (p["launches"], p["workgroups"]) == (2, 2 * ((1 << 20) + 1))
    # just below the limit: one launch
    st, p = _plan_ex(g, RI, shape=(1024, 1), rows=1 << 21, width=G, group_size=G,
                     y_row_stride=G, gate_row_stride=G, out_row_stride=G, gate=A + (1 << 26),
                     norm_weight=A + (2 << 26), out=A + (3 << 26))
    assert st == OK and p["launches"] == 1


def test_vector_width_follows_alignment(g):
    assert _plan(g, 4, 256, 64, BF16)["vector_bytes"] == 16
    assert _plan(g, 4, 256, 64, BF16, y=A + 8)["vector_bytes"] == 8
    assert _plan(g, 4, 256, 64, BF16, out=A + (3 << 30) + 4)["vector_bytes"] == 4
    assert _plan(g, 4, 256, 64, BF16, y=A + 2)["vector_bytes"] == 2
    assert _plan(g, 4, 258, 258, BF16, sy=258, sg=258, so=258)["vector_bytes"] == 4
    assert _plan(g, 4, 256, 64, BF16, sy=260)["vector_bytes"] == 8
    assert _plan(g, 3, 63 * 5, 63, BF16)["vector_bytes"] == 2
    # the weight loads must be aligned for the matching width too
    # (two bf16 per 4-byte vector take an 8-byte weight load, so a 4-byte
    # aligned weight leaves one element per access)
    assert _plan(g, 4, 256, 64, BF16, w=A + (2 << 30) + 4)["vector_bytes"] == 2
    assert _plan(g, 4, 256, 64, F32, w=A + (2 << 30) + 4)["vector_bytes"] == 4


def test_kernel_family_by_group_width(g):
    """The measured shape table: (kernel, lanes, vectors per lane, rows per
    workgroup) by 16-byte vectors per group."""
    cases = {
        8: ("wave", 1, 1, 1),         # 1 vector: a group per lane
        64: ("wave", 8, 1, 1),
        512: ("wave", 64, 1, 1),      # 64
        576: ("wave", 64, 2, 1),      # 72
        640: ("wave", 64, 2, 1),      # 80
        648: ("block", 128, 1, 1),    # 81
        768: ("block", 128, 1, 1),    # 96
        776: ("block", 128, 1, 2),    # 97
        832: ("block", 128, 1, 2),    # 104
        840: ("block", 128, 1, 4),    # 105
        960: ("block", 128, 1, 4),    # 120
        1032: ("block", 128, 2, 2),   # 129
        1152: ("block", 128, 2, 2),   # 144
        1160: ("block", 128, 2, 4),   # 145
        1536: ("block", 128, 2, 4),   # 192
        2048: ("block", 256, 1, 2),   # 256
        2056: ("block", 128, 3, 2),   # 257
        4096: ("block", 256, 2, 2),   # 512
        5120: ("block", 256, 3, 1),   # 640
        6144: ("block", 256, 3, 1),   # 768
        6152: ("block", 256, 4, 1),   # 769
        7680: ("block", 256, 4, 1),   # 960
        12288: ("block", 256, 6, 1),  # 1536
        12296: ("block", 512, 4, 1),  # 1537
        16384: ("block", 512, 4, 1),  # 2048
        24576: ("block", 1024, 3, 1),  # 3072
        32768: ("block", 1024, 4, 1),
        32776: ("wide", 1024, 0, 1),
    }
    for G, want in cases.items():
        p = _plan(g, 8, G, G, BF16)
        got = (p["kernel_name"], p["lanes_per_group"], p["vectors_per_lane"], p["rows_per_workgroup"])
        assert got == want, (G, got)
    # rows per workgroup never exceeds the rows there are
    assert _plan(g, 1, 960, 960, BF16)["rows_per_workgroup"] == 1
    assert _plan(g, 3, 960, 960, BF16)["rows_per_workgroup"] == 2


def test_division_magic_numbers(tmp_path):
    """unit / groups by multiply-high: exhaustive small divisors and dividends,
    plus random large ones, against integer division."""
    drv = tmp_path / "divcheck.cpp"
    drv.write_text(r'''
#include <cstdint>
#include <cstdio>
#include <random>
#include "ggrms_internal.h"
static uint32_t q(uint32_t n, uint32_t m, uint32_t s) {
    return (uint32_t)((((uint64_t)n * m) >> 32) + n) >> s;
}
int main() {
    std::mt19937_64 rng(1);
    for (uint32_t d = 1; d < 5000; ++d) {
        uint32_t m, s; ggrms::div_magic(d, &m, &s);
        for (uint32_t n = 0; n < 20000; ++n) if (q(n, m, s) != n / d) { printf("%u %u\n", n, d); return 1; }
        for (int i = 0; i < 2000; ++i) { uint32_t n = rng() & 0x7FFFFFFF; if (q(n, m, s) != n / d) { printf("%u %u\n", n, d); return 1; } }
    }
    for (int i = 0; i < 200000; ++i) {
        uint32_t d = (uint32_t)(rng() % 0x7FFFFFFF) + 1, n = rng() & 0x7FFFFFFF, m, s;
        ggrms::div_magic(d, &m, &s);
        if (q(n, m, s) != n / d) { printf("%u %u\n", n, d); return 1; }
        n = 0x7FFFFFFF; if (q(n, m, s) != n / d) { printf("%u %u\n", n, d); return 1; }
    }
    return 0;
}
''')
    exe = tmp_path / "divcheck"
    csrc = os.path.join(ROOT, "gated_group_rmsnorm_amd", "csrc")
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I", csrc,
                    str(drv), os.path.join(csrc, "plan.cpp"), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout


def test_planner_host_sanitizers(tmp_path):
    """The planner (pure host C++) under AddressSanitizer and UBSan over a
    sweep of shapes, strides and pointers, and of packed layouts (runs,
    shared weights, forced shapes)."""
    drv = tmp_path / "plansweep.cpp"
    drv.write_text(r'''
#include <cstdint>
#include <cstdio>
#include <initializer_list>
#include "ggrms.h"
#include "ggrms_tuning.h"
int main() {
    const int64_t Gs[] = {1, 2, 3, 7, 8, 63, 64, 65, 100, 128, 960, 4096, 7680, 32768, 65536};
    const uintptr_t base = 1u << 20;
    long n_ok = 0;
    for (int64_t G : Gs) for (int64_t rows : {0, 1, 3, 257}) for (int dt = 0; dt < 4; ++dt)
    for (int off = 0; off < 3; ++off) {
        ggrms_plan_t p;
        int64_t width = G * 3;
        ggrms_status_t st = ggrms_plan((void*)(base + off * 2), (void*)(base + (1u << 28)),
                                       (const float*)(base + (2u << 28)), (void*)(base + (3u << 28)),
                                       rows, width, G, width + off, width, width, 1e-5f,
                                       (ggrms_dtype_t)dt, 1, &p);
        n_ok += st == GGRMS_SUCCESS;
        const ggrms_shape_t shapes[] = {{64, 2, 0, 0}, {128, 1, 4, 0}, {256, 3, 2, 0},
                                        {1024, 0, 0, 0}, {16, 1, 0, 0}, {0, 0, 0, 0},
                                        {128, 1, -1, 0}, {0, 0, 0, 8}, {0, 0, 0, 4},
                                        {512, 1, 0, 4}, {0, 0, 0, 3}, {64, 1, 0, 16}};
        for (uint32_t flags = 0; flags < 520; flags += (flags < 40 ? 1 : 31)) {
            st = ggrms_plan_ex((void*)(base + off * 2), (void*)(base + (1u << 28)),
                               (const float*)(base + (2u << 28) + off * 4),
                               (void*)(base + (3u << 28)), rows, width, G, width + off, width,
                               width, 1e-5f, (ggrms_dtype_t)dt, flags, &p);
            n_ok += st == GGRMS_SUCCESS;
            for (const ggrms_shape_t& sh : shapes) {
                st = ggrms_plan_tuned((void*)(base + off * 2), (void*)(base + (1u << 28)),
                                      (const float*)(base + (2u << 28)),
                                      (void*)(base + (3u << 28)), rows, width, G, width + off,
                                      width, width, 1e-5f, (ggrms_dtype_t)dt, flags, &sh, &p);
                n_ok += st == GGRMS_SUCCESS;
            }
            // out over the weight, and over the gap of a strided row
            st = ggrms_plan_ex((void*)(base + off * 2), (void*)(base + (1u << 28)),
                               (const float*)(base + (2u << 28)),
                               (void*)(base + (2u << 28) - 2 * width * (off + 1)), rows, width,
                               G, width + off, width, 3 * width, 1e-5f, (ggrms_dtype_t)dt,
                               flags & 7, &p);
            n_ok += st == GGRMS_SUCCESS;
        }
    }
    // packed groups (16-byte aligned rows of groups that are not a whole
    // number of vectors): runs by default and forced, shared weights, ROWS
    const int64_t Ps[] = {9, 13, 25, 99, 100, 127, 180, 230, 250, 300, 513, 1001, 4099};
    for (int64_t G : Ps) for (int64_t rows : {1, 5, 3000, 30000}) for (int dt = 0; dt < 3; ++dt)
    for (uint32_t flags : {0u, 1u, 2u, 4u, 5u, 6u, 33u, 65u, 257u}) {
        ggrms_plan_t p;
        const int64_t width = G * 16;
        const ggrms_shape_t shapes[] = {{0, 0, 0, 0, GGRMS_KERNEL_RUN}, {64, 1, 0, 0, GGRMS_KERNEL_RUN},
                                        {64, 2, 0, 0, GGRMS_KERNEL_RUN}, {64, 3, 0, 0, GGRMS_KERNEL_RUN},
                                        {0, 0, 0, 0, GGRMS_KERNEL_ROWS}, {16, 1, 0, 0, 0},
                                        {8, 2, 0, 0, 0}, {0, 0, 0, 0, 0}};
        for (int woff : {0, 4, 8})
        for (const ggrms_shape_t& sh : shapes) {
            ggrms_status_t st = ggrms_plan_tuned(
                (void*)base, (void*)(base + (1u << 28)), (const float*)(base + (2u << 28) + woff),
                (void*)(base + (3u << 28)), rows, width, G, width, width, width, 1e-5f,
                (ggrms_dtype_t)dt, flags, &sh, &p);
            n_ok += st == GGRMS_SUCCESS;
        }
    }
    printf("%ld\n", n_ok);
    return n_ok > 0 ? 0 : 1;
}
''')
    exe = tmp_path / "plansweep"
    csrc = os.path.join(ROOT, "gated_group_rmsnorm_amd", "csrc")
    subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-I", csrc,
                    str(drv), os.path.join(csrc, "plan.cpp"), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr


C_CLIENT = r"""
#include <stdint.h>
#include <stdio.h>
#include "ggrms.h"

int main(void) {
    /* fake, 256-byte aligned device addresses: planning makes no HIP call */
    const void* y = (const void*)(uintptr_t)0x100000;
    const void* gate = (const void*)(uintptr_t)0x4100000;
    const float* w = (const float*)(uintptr_t)0x8100000;
    void* out = (void*)(uintptr_t)0xc100000;
    ggrms_plan_t p;
    ggrms_status_t st = ggrms_plan(y, gate, w, out, 8192, 7680, 960, 7680, 7680, 7680, 1e-5f,
                                   GGRMS_BF16, 1, &p);
    /* rejected before any HIP call: width is not a multiple of the group */
    ggrms_status_t bad = ggrms_forward(y, gate, w, out, 4, 1000, 960, 1000, 1000, 1000, 1e-5f,
                                       GGRMS_BF16, 1, NULL);
    printf("%d %d %d %d %d %lld %d %s\n", ggrms_abi_version(), (int)st, p.kernel,
           p.lanes_per_group, p.rows_per_workgroup, (long long)p.workgroups, (int)bad,
           ggrms_status_string(bad));
    return st == GGRMS_SUCCESS && bad == GGRMS_ERROR_INVALID_VALUE ? 0 : 1;
}
"""


@pytest.mark.parametrize("compiler", [["gcc", "-x", "c", "-std=c99"], ["g++", "-x", "c++", "-std=c++11"]],
                         ids=["c99", "c++11"])
def test_c_client_builds_and_links(g, tmp_path, compiler):
    """The header is plain C (and C++): a client compiled with -pedantic
    -Werror links against the library and plans the prefill job through the
    C ABI alone."""
    src = tmp_path / "client.c"
    src.write_text(C_CLIENT)
    exe = tmp_path / "client"
    libdir = os.path.dirname(g.library_path())
    subprocess.run([*compiler, "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-I", os.path.join(ROOT, "include"), str(src), "-x", "none",
                    "-L", libdir, "-l:libggrms.so", f"-Wl,-rpath,{libdir}", "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    fields = r.stdout.split()
    assert fields[:7] == [str(g.ABI_VERSION), "0", "2", "128", "4", str(8192 // 4 * 8), "1"], r.stdout
    assert " ".join(fields[7:]) == g.ggrms_status_string(1)


def test_weight_spellings_for_the_torch_wrapper(g):
    """forward()'s weight handling on the CPU: (n), (1, n) and (n, 1) in f32,
    fp16 or bf16 become the same contiguous f32 vector (16-bit values widen
    exactly); other shapes, lengths and dtypes are refused."""
    import torch

    base = torch.arange(1, 129, dtype=torch.float32) / 64  # exact in fp16 and bf16
    for t in (base, base.reshape(1, 128), base.reshape(128, 1), base.half(),
              base.bfloat16().reshape(1, 128), base.reshape(128, 1).half()):
        w = g._weight_f32(t, 1024, 128)
        assert w.dtype == torch.float32 and w.dim() == 1 and w.is_contiguous()
        assert torch.equal(w, base), tuple(t.shape)
    # a non-contiguous column of a wider tensor is copied out
    wide = torch.stack([base, -base], dim=1)  # [128, 2]
    assert torch.equal(g._weight_f32(wide[:, :1], 1024, 128), base)
    assert g._weight_f32(torch.ones(1024), 1024, 128).numel() == 1024
    with pytest.raises(ValueError):
        g._weight_f32(base.reshape(2, 64), 1024, 128)
    with pytest.raises(ValueError):
        g._weight_f32(base.reshape(1, 1, 128), 1024, 128)
    with pytest.raises(ValueError):
        g._weight_f32(base[:100], 1024, 128)
    with pytest.raises(TypeError):
        g._weight_f32(base.double(), 1024, 128)
