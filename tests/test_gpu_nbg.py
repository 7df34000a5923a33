"""GPU parity of the operator variants against the CPU oracle: norm before
gate (page "com.microsoft.GatedRMSNorm", Description section: the RMS of y
alone, then the scale, then silu(gate)) and a weight of group_size values
shared by every group (that page's `scale` input), each through
ggrms_forward_ex (ggrms_forward_tuned where a shape or a launch control is
forced).

Same bar as the gate-first tests: f32 within a relative 1e-5 of the oracle,
fp16/bf16 within 2 units in the last place, NaN where the oracle has NaN.
"""
import math

import numpy as np
import pytest
import torch

import refs
import synthetic as S
from gpu_util import (BF16, DT_IDS, F16, F32, FLAG_NBG, FLAG_PER_GROUP, FLAG_RI, TDT,
                      assert_parity, check_contiguous, dev_buf, host_bits, random_case, run_gpu,
                      say)

pytestmark = pytest.mark.gpu

NBG, NBG_PG = FLAG_NBG, FLAG_NBG | FLAG_PER_GROUP


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


def workload_weight(w, wt):
    """The workload's weight in the form its operator takes: the per-head
    scale itself where the workload has one spanning a group, else the
    per-column weight."""
    if w.scale_len and w.scale_len == w.group_size:
        return np.ascontiguousarray(wt[:w.group_size]), True
    return wt, False


@pytest.mark.parametrize("name", list(S.WORKLOADS))
def test_workload_full_size_nbg(g, orc, name):
    """Every configured workload at full size in the norm-first operator,
    element by element, in the benchmark's layout; the 128-wide fp16 head
    scale of the GDN-shaped workload is passed as the shared group weight."""
    w = S.WORKLOADS[name]
    ybuf, gbuf, wt, lay = S.make_inputs(w)
    wt, per_group = workload_weight(w, wt)
    say(f"workload {name} nbg per_group={per_group}")
    rows, width = w.rows, w.width
    wd = torch.from_numpy(wt).cuda()
    if w.fused_width:
        fd = dev_buf(ybuf, w.dtype)
        yv, gv = fd[lay["y_offset"]:], fd[lay["gate_offset"]:]
    else:
        yv, gv = dev_buf(ybuf, w.dtype), dev_buf(gbuf, w.dtype)
    od = torch.empty(rows * width, dtype=TDT[w.dtype], device="cuda")
    flags = NBG | (FLAG_PER_GROUP if per_group else 0)
    st = run_gpu(g, yv, gv, wd, od, rows, width, w.group_size, lay["y_row_stride"],
                 lay["gate_row_stride"], width, w.eps, w.dtype, 0, flags=flags)
    assert st == g.SUCCESS, g.ggrms_status_string(st)
    torch.cuda.synchronize()
    got = host_bits(od, w.dtype)
    ref = orc.forward(ybuf, gbuf, wt, rows=rows, width=width, group_size=w.group_size,
                      y_row_stride=lay["y_row_stride"], gate_row_stride=lay["gate_row_stride"],
                      out_row_stride=width, eps=w.eps, dtype=w.dtype, y_offset=lay["y_offset"],
                      gate_offset=lay["gate_offset"], norm_before_gate=True,
                      weight_per_group=per_group)
    stats = assert_parity(got, ref, w.dtype, name)
    say(f"  {name} nbg: {stats}")


G_SWEEP = [1, 3, 8, 24, 63, 64, 100, 128, 129, 257, 960, 1024, 2056, 4096, 7680, 32768, 32776]


def _nbg_wide_f32_against_exact(g, orc, G, flags):
    """f32 groups wider than 4096, norm first: the GPU against the exact
    result (library routines in float64, tests/refs.py) within 1e-5, and the
    oracle against it within its own f32 bound ((G/2 + 16) * 2^-24 relative),
    since the oracle's sequential sum may itself be ~1e-5 off at these widths."""
    rows, groups = 3, 2
    width = G * groups
    say(f"case nbg wide f32 G={G} flags={flags} against the float64 chain")
    y, gt, w = random_case(rows, width, F32, seed=G * 5 + F32 + flags)
    if flags & FLAG_PER_GROUP:
        w = np.ascontiguousarray(w[:G])
    yd, gd, wd = dev_buf(y, F32), dev_buf(gt, F32), torch.from_numpy(w).cuda()
    od = torch.empty_like(yd)
    assert run_gpu(g, yd, gd, wd, od, rows, width, G, width, width, width, 1e-5, F32, 0,
                   flags=flags) == g.SUCCESS
    torch.cuda.synchronize()
    got = host_bits(od, F32).reshape(rows, width).astype(np.float64)
    wcol = np.tile(w, groups) if flags & FLAG_PER_GROUP else w
    ref = refs.chain_nbg_fp64(y.reshape(rows, width).astype(np.float64),
                              gt.reshape(rows, width).astype(np.float64),
                              wcol.astype(np.float64), G, float(np.float32(1e-5)))
    rel = np.abs(got - ref) / np.maximum(np.abs(ref), 1e-38)
    assert rel.max() <= 1e-5, f"G={G}: GPU off the exact result by {rel.max():.3e} relative"
    o = orc.forward(y, gt, w, rows=rows, width=width, group_size=G, y_row_stride=width,
                    gate_row_stride=width, out_row_stride=width, eps=1e-5, dtype=F32,
                    round_intermediate=0, norm_before_gate=True,
                    weight_per_group=bool(flags & FLAG_PER_GROUP)).reshape(rows, width)
    orel = np.abs(o.astype(np.float64) - ref) / np.maximum(np.abs(ref), 1e-38)
    assert orel.max() <= refs.oracle_delta(G), f"G={G}: oracle off the exact result by {orel.max():.3e}"


@pytest.mark.parametrize("dtype", [BF16, F16, F32], ids=DT_IDS.get)
@pytest.mark.parametrize("G", G_SWEEP)
def test_nbg_group_size_sweep(g, orc, G, dtype):
    """The norm-first operator on every kernel family (one group per lane,
    wave segments, multi-wave workgroups with staged weights, the two-pass
    kernel), with per-column and shared group weights."""
    if dtype == F32 and G > 4096:
        for flags in (NBG, NBG_PG):
            _nbg_wide_f32_against_exact(g, orc, G, flags)
        return
    groups = 3 if G <= 4096 else 2
    rows = 6 if G <= 1024 else 3
    for flags in (NBG, NBG_PG):
        check_contiguous(g, orc, rows, G * groups, G, dtype, 0, seed=G * 5 + dtype + flags,
                         tag=f"nbg G={G}", flags=flags)


@pytest.mark.parametrize("dtype", [BF16, F16, F32], ids=DT_IDS.get)
@pytest.mark.parametrize("G", [8, 100, 960, 2056, 32776])
def test_shared_weight_equals_tiled_weight(g, orc, G, dtype):
    """A shared group weight gives the same bits as the same values tiled
    over every group as a per-column weight, in both operators."""
    groups, rows = 3, 5
    width = G * groups
    y, gt, w = random_case(rows, width, dtype, seed=G + 3 * dtype)
    wg = np.ascontiguousarray(w[:G])
    yd, gd = dev_buf(y, dtype), dev_buf(gt, dtype)
    wgd = torch.from_numpy(wg).cuda()
    wtd = torch.from_numpy(np.tile(wg, groups)).cuda()
    for base in ((0, FLAG_RI) if dtype != F32 else (0,)) + (FLAG_NBG,):
        say(f"case shared weight G={G} dtype={DT_IDS[dtype]} base={base}")
        o1, o2 = torch.empty_like(yd), torch.empty_like(yd)
        assert run_gpu(g, yd, gd, wgd, o1, rows, width, G, width, width, width, 1e-5, dtype, 0,
                       flags=base | FLAG_PER_GROUP) == g.SUCCESS
        assert run_gpu(g, yd, gd, wtd, o2, rows, width, G, width, width, width, 1e-5, dtype, 0,
                       flags=base) == g.SUCCESS
        torch.cuda.synchronize()
        a, b = host_bits(o1, dtype), host_bits(o2, dtype)
        assert np.array_equal(a.view(np.uint32) if dtype == F32 else a,
                              b.view(np.uint32) if dtype == F32 else b)
        ref = orc.forward(y, gt, wg, rows=rows, width=width, group_size=G, y_row_stride=width,
                          gate_row_stride=width, out_row_stride=width, eps=1e-5, dtype=dtype,
                          round_intermediate=base & FLAG_RI,
                          norm_before_gate=bool(base & FLAG_NBG), weight_per_group=True)
        assert_parity(a, ref, dtype, f"shared weight base={base}")


SHAPES = [(1, 1), (4, 1), (16, 1), (64, 1), (64, 2), (64, 4)] + \
         [(l, v, 1) for l in (128, 256, 512, 1024) for v in (1, 4)] + \
         [(128, v, u) for v in (1, 2) for u in (2, 4)] + [(256, 2, 2), (1024, 0)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_nbg_forced_shapes(g, orc, shape):
    """Each kernel shape, forced, in the norm-first operator with a shared
    group weight (the staged-weight path reads the same G values for every
    group), on 7 rows so the last row tile is partly empty."""
    lanes, vpt = shape[:2]
    cap = lanes * (vpt or 8)
    for nvec in sorted({max(1, cap), max(1, cap - 3)}):
        G = nvec * 8
        if G > 65536:
            continue
        for flags in (NBG, NBG_PG):
            check_contiguous(g, orc, 7, G * 2, G, BF16, 0, seed=nvec + lanes + flags,
                             shape=shape, tag=f"nbg forced {shape} G={G}", flags=flags)


@pytest.mark.parametrize("dtype", [BF16, F16, F32], ids=DT_IDS.get)
def test_nbg_special_values(g, orc, dtype):
    """NaN/inf in y (the whole group follows) and in the gate (only that
    element: silu(gate) multiplies after the norm), zero groups, gates in
    silu's underflow window and large gates."""
    rows, width, G = 16, 1024, 128
    rng = np.random.default_rng(19)
    yv = rng.standard_normal((rows, width))
    gv = rng.standard_normal((rows, width))
    yv[0, 5] = np.nan
    yv[1, 200] = np.inf
    gv[2, 300] = np.nan
    yv[3, :G] = 0.0
    gv[4, :] = rng.uniform(-104, -86, width)
    gv[5, :G] = -95.0
    gv[6, :] = rng.uniform(80, 100, width)
    gv[7, 7] = -np.inf
    gv[7, 300] = np.inf
    yv[8, G:2 * G] = 1e-30  # tiny but non-zero: nf large, products near the range's ends
    import refs
    y = refs.round64(yv, dtype).reshape(-1)
    gt = refs.round64(gv, dtype).reshape(-1)
    w = rng.uniform(0.5, 1.5, width).astype(np.float32)
    yd, gd = dev_buf(y, dtype), dev_buf(gt, dtype)
    for per_group in (False, True):
        wa = np.ascontiguousarray(w[:G]) if per_group else w
        wd = torch.from_numpy(wa).cuda()
        for eps in (1e-5, 0.0):
            say(f"case nbg special dtype={DT_IDS[dtype]} eps={eps} per_group={per_group}")
            od = torch.empty_like(yd)
            flags = NBG_PG if per_group else NBG
            assert run_gpu(g, yd, gd, wd, od, rows, width, G, width, width, width, eps, dtype, 0,
                           flags=flags) == g.SUCCESS
            torch.cuda.synchronize()
            ref = orc.forward(y, gt, wa, rows=rows, width=width, group_size=G,
                              y_row_stride=width, gate_row_stride=width, out_row_stride=width,
                              eps=eps, dtype=dtype, norm_before_gate=True,
                              weight_per_group=per_group)
            assert_parity(host_bits(od, dtype), ref, dtype, f"nbg special eps={eps}")


def test_nbg_strided_and_in_place(g, orc):
    """Column slices of one fused buffer with padded strides, and the output
    written over the gate, in the norm-first operator."""
    rows, width, G, fused = 37, 4800, 100, 9856
    buf = S.tensor(41, S.TID_Y, rows * fused, F16, ("normal", 1.0))
    w = S.tensor(41, S.TID_W, G, F32, ("uniform", 0.5, 1.5))
    ref = orc.forward(buf, buf, w, rows=rows, width=width, group_size=G, y_row_stride=fused,
                      gate_row_stride=fused, out_row_stride=fused, eps=1e-5, dtype=F16,
                      gate_offset=width, out_offset=width, norm_before_gate=True,
                      weight_per_group=True, out=buf.copy())
    fd = dev_buf(buf, F16)
    wd = torch.from_numpy(w).cuda()
    say("case nbg strided in place")
    assert run_gpu(g, fd, fd[width:], wd, fd[width:], rows, width, G, fused, fused, fused, 1e-5,
                   F16, 0, flags=NBG_PG) == g.SUCCESS
    torch.cuda.synchronize()
    assert_parity(host_bits(fd, F16), ref, F16, "nbg strided in place")


def test_nbg_rejections(g):
    """Round-intermediate with norm-first, both cache policies at once, both
    tile orders or both WAVE workgroup sizes at once, and unknown flag bits
    are refused before any launch; the output is left untouched."""
    yd = torch.ones(4 * 256, dtype=torch.bfloat16, device="cuda")
    wd = torch.ones(256, dtype=torch.float32, device="cuda")
    od = torch.full_like(yd, 7.0)
    for flags in (FLAG_RI | FLAG_NBG, 8 | 16, 32 | 64, 128 | 256, 512, 1 << 20):
        assert run_gpu(g, yd, yd, wd, od, 4, 256, 64, 256, 256, 256, 1e-5, BF16, 0,
                       flags=flags) == g.ERROR_INVALID_VALUE
    torch.cuda.synchronize()
    assert bool((od == 7.0).all())


def test_nbg_graph_capture_replays(g, orc):
    """21 decode-sized norm-first launches (shared 960-value weight) captured
    once and replayed with eager work between replays: every layer of the
    eager burst meets the bar against the oracle, and each replay equals the
    eager result bit for bit."""
    width, G = 7680, 960
    layers, refs_ = [], []
    for layer in range(S.DECODE_LAYERS):
        y, gt, w = random_case(1, width, BF16, seed=500 + layer)
        wg = np.ascontiguousarray(w[:G])
        layers.append((dev_buf(y, BF16), dev_buf(gt, BF16), torch.from_numpy(wg).cuda(),
                       torch.empty(width, dtype=torch.bfloat16, device="cuda")))
        refs_.append(orc.forward(y, gt, wg, rows=1, width=width, group_size=G,
                                 y_row_stride=width, gate_row_stride=width, out_row_stride=width,
                                 eps=1e-5, dtype=BF16, round_intermediate=0,
                                 norm_before_gate=True, weight_per_group=True))
    torch.cuda.synchronize()

    def burst(stream):
        for yd, gd, wd, od in layers:
            assert run_gpu(g, yd, gd, wd, od, 1, width, G, width, width, width, 1e-5, BF16, 0,
                           stream=stream, flags=NBG_PG) == g.SUCCESS

    burst(torch.cuda.current_stream())
    torch.cuda.synchronize()
    eager = [o.clone() for *_, o in layers]
    for layer, (e, ref) in enumerate(zip(eager, refs_)):
        assert_parity(host_bits(e, BF16), ref, BF16, f"norm-first decode layer {layer}")
    graph = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    with torch.cuda.graph(graph, stream=cs):
        burst(cs)
    for rep in range(3):
        for *_, o in layers:
            o.fill_(0)
        junk = torch.randn(1 << 20, device="cuda").sum()
        graph.replay()
        torch.cuda.synchronize()
        assert junk.isfinite()
        for o, e in zip((o for *_, o in layers), eager):
            assert torch.equal(o.view(torch.int16), e.view(torch.int16)), f"replay {rep}"


def test_torch_wrapper_nbg(g, orc):
    """forward(norm_before_gate=True) with the per-head scale passed as is
    (group_size values) and tiled (width values) gives the same bits and
    matches the oracle; round_intermediate with it raises."""
    B, T, H, C = 3, 7, 16, 128
    width = H * C
    fused = torch.randn(B, T, 2 * width, generator=torch.Generator().manual_seed(3)).to(torch.float16)
    scale = (torch.rand(C, generator=torch.Generator().manual_seed(4)) + 0.5).to(torch.float16)
    fd = fused.cuda()
    y, gate = fd[..., :width], fd[..., width:]
    w_head = scale.float().cuda()
    o1 = g.forward(y, gate, w_head, C, eps=1e-6, norm_before_gate=True)
    o2 = g.forward(y, gate, g.expand_head_scale(scale.cuda(), H), C, eps=1e-6,
                   norm_before_gate=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    yh = fused[..., :width].contiguous().view(torch.int16).numpy().view(np.uint16).reshape(-1)
    gh = fused[..., width:].contiguous().view(torch.int16).numpy().view(np.uint16).reshape(-1)
    ref = orc.forward(yh, gh, scale.float().numpy(), rows=B * T, width=width, group_size=C,
                      y_row_stride=width, gate_row_stride=width, out_row_stride=width, eps=1e-6,
                      dtype=F16, norm_before_gate=True, weight_per_group=True)
    assert_parity(o1.cpu().view(torch.int16).numpy().view(np.uint16).reshape(-1), ref, F16,
                  "wrapper nbg")
    with pytest.raises(g.GgrmsError):
        g.forward(y, gate, w_head, C, round_intermediate=True, norm_before_gate=True)
    assert g.plan(y, gate, w_head, C, norm_before_gate=True)["kernel_name"] == "wave"


PACKED_SHARED_CASES = [(100, F16), (99, BF16), (127, BF16), (250, F16), (13, F16), (9, BF16),
                       (1001, BF16), (25, F32), (99, F32)]


@pytest.mark.parametrize("G,dtype", PACKED_SHARED_CASES,
                         ids=[f"G{G}-{DT_IDS[d]}" for G, d in PACKED_SHARED_CASES])
def test_packed_groups_shared_weight(g, orc, G, dtype):
    """Packed groups (byte length not a multiple of 16, rows that are) with one
    weight of group_size values shared by every group, read piece by piece
    on lane segments or staged in LDS by runs of groups (the library's run,
    one and two vectors per lane): both operators, row-major and banded order
    (same bits), out rows padded and guarded, nothing outside the view
    written; a weight 4 bytes past an alignment boundary too (packed where a
    piece's weights are one float, narrower vectors otherwise)."""
    groups, rows = 16, (5 if G <= 1001 else 3)
    width = G * groups
    esz = 4 if dtype == F32 else 2
    so = width + 16 // esz
    guard = 64
    y, gt, _ = random_case(rows, width, dtype, seed=G * 11 + dtype)
    w = S.tensor(G * 11 + dtype, S.TID_W, G, F32, ("uniform", 0.5, 1.5))
    canary = {F32: np.float32(-1234.5), F16: np.uint16(0x7BFF), BF16: np.uint16(0x4B4B)}[dtype]
    ob = np.full(guard + (rows - 1) * so + width + guard, canary, dtype=S.storage_dtype(dtype))
    view = np.zeros(ob.shape, dtype=bool)
    for r in range(rows):
        view[guard + r * so: guard + r * so + width] = True
    yd, gd = dev_buf(y, dtype), dev_buf(gt, dtype)
    wbuf = torch.zeros(G + 1, dtype=torch.float32, device="cuda")
    wbuf[1:] = torch.from_numpy(w).cuda()
    w_off = wbuf[1:]                       # 4 bytes past an allocation boundary
    w_al = torch.from_numpy(w).cuda()      # aligned as allocated
    pe = math.gcd(G * esz, 16) // esz      # weights per piece
    gate_first = FLAG_RI if dtype != F32 else 0
    for wd, base in ((w_al, gate_first), (w_off, gate_first), (w_al, FLAG_NBG), (w_off, FLAG_NBG)):
        flags = base | FLAG_PER_GROUP
        ref = orc.forward(y, gt, w, rows=rows, width=width, group_size=G, y_row_stride=width,
                          gate_row_stride=width, out_row_stride=so, eps=1e-5, dtype=dtype,
                          round_intermediate=base & FLAG_RI, norm_before_gate=bool(base & FLAG_NBG),
                          weight_per_group=True, out=ob.copy(), out_offset=guard)
        aligned = wd.data_ptr() % (4 * pe) == 0
        # the library's shape, and runs of groups with the weight staged in LDS
        shapes = [None] + ([(0, 0, 0, 0, g.KERNEL_RUN), (64, 1, 0, 0, g.KERNEL_RUN),
                            (64, 2, 0, 0, g.KERNEL_RUN)] if aligned and G <= 512 else [])
        for shape in shapes:
            outs = []
            for order in (0, 32, 64):  # the library's order, row-major, banded
                od = dev_buf(ob, dtype)
                st, p = g.ggrms_plan_tuned(yd.data_ptr(), gd.data_ptr(), wd.data_ptr(),
                                           od[guard:].data_ptr(), rows, width, G, width, width, so,
                                           1e-5, dtype, flags | order, shape)
                if shape is not None and st == g.ERROR_NOT_SUPPORTED:
                    break  # two groups do not fit one vector per lane
                assert st == g.SUCCESS and (p["vector_bytes"] == 16 and p["piece_bytes"] < 16) == \
                    aligned, p
                say(f"case packed shared weight G={G} dtype={DT_IDS[dtype]} flags={flags} "
                    f"order={order} {p['kernel_name']} {p['lanes_per_group']}x"
                    f"{p['vectors_per_lane']} runs of {p['groups_per_run']}")
                assert run_gpu(g, yd, gd, wd, od[guard:], rows, width, G, width, width, so, 1e-5,
                               dtype, 0, shape=shape, flags=flags | order) == g.SUCCESS
                torch.cuda.synchronize()
                got = host_bits(od, dtype)
                assert np.array_equal(got[~view].view(np.uint8), ob[~view].view(np.uint8)), \
                    "stores touched elements outside the view"
                outs.append(got)
            if not outs:
                continue
            assert all(np.array_equal(o.view(np.uint8), outs[0].view(np.uint8)) for o in outs[1:])
            assert_parity(outs[0][view], ref[view], dtype,
                          f"packed shared G={G} flags={flags} shape={shape}")
