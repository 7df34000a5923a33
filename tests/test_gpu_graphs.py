"""GPU: every kernel family is safe to capture into a HIP graph.

The entry points allocate nothing, never synchronise and record no memset, so
a caller may capture them.  One graph holds launches of each kernel family --
lane segments over packed groups, runs of packed groups with a shared weight
staged in LDS (dynamic LDS), BLOCK with weights staged for four rows, ROWS,
the two-pass WIDE kernel, and the norm-first operator -- and is replayed
several times with eager work and a clear of every output between replays.
The eager launches meet the bar against the oracle, and every replay equals
the eager outputs bit for bit.
"""
import numpy as np
import pytest
import torch

from gpu_util import (BF16, F16, FLAG_NBG, FLAG_PER_GROUP, FLAG_RI, assert_parity, dev_buf,
                      host_bits, random_case, run_gpu, say)

pytestmark = pytest.mark.gpu

KERNEL_RUN, KERNEL_ROWS = 4, 5

# (label, rows, groups, G, dtype, flags, forced shape, expected kernel)
JOBS = [
    ("packed segments", 64, 48, 100, F16, FLAG_RI, None, "wave"),
    ("runs, shared weight", 32, 16, 127, BF16, FLAG_RI | FLAG_PER_GROUP,
     (0, 0, 0, 0, KERNEL_RUN), "run"),
    ("block, staged weights", 64, 8, 960, BF16, FLAG_RI, None, "block"),
    ("rows", 300, 1, 5120, BF16, FLAG_RI, (0, 0, 0, 0, KERNEL_ROWS), "rows"),
    ("wide", 3, 1, 40960, BF16, FLAG_RI, None, "wide"),
    ("norm first, shared weight", 48, 16, 128, F16, FLAG_NBG | FLAG_PER_GROUP, None, "wave"),
]


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


def test_kernel_families_replay_from_one_graph(g, orc):
    cases = []
    for i, (label, rows, groups, G, dtype, flags, shape, kname) in enumerate(JOBS):
        width = G * groups
        y, gt, w = random_case(rows, width, dtype, seed=9700 + i)
        if flags & FLAG_PER_GROUP:
            w = np.ascontiguousarray(w[:G])
        yd, gd, wd = dev_buf(y, dtype), dev_buf(gt, dtype), torch.from_numpy(w).cuda()
        od = torch.empty_like(yd)
        st, p = g.ggrms_plan_tuned(yd.data_ptr(), gd.data_ptr(), wd.data_ptr(), od.data_ptr(),
                                   rows, width, G, width, width, width, 1e-5, dtype, flags, shape)
        assert st == g.SUCCESS and p["kernel_name"] == kname, (label, p)
        ref = orc.forward(y, gt, w, rows=rows, width=width, group_size=G, y_row_stride=width,
                          gate_row_stride=width, out_row_stride=width, eps=1e-5, dtype=dtype,
                          round_intermediate=flags & FLAG_RI,
                          norm_before_gate=bool(flags & FLAG_NBG),
                          weight_per_group=bool(flags & FLAG_PER_GROUP))
        cases.append((label, rows, width, G, dtype, flags, shape, yd, gd, wd, od, ref))

    def launch_all(stream):
        for label, rows, width, G, dtype, flags, shape, yd, gd, wd, od, _ in cases:
            st = run_gpu(g, yd, gd, wd, od, rows, width, G, width, width, width, 1e-5, dtype, 0,
                         shape=shape, stream=stream, flags=flags)
            assert st == g.SUCCESS, (label, g.ggrms_status_string(st))

    say("case graph of kernel families: eager")
    launch_all(torch.cuda.current_stream())
    torch.cuda.synchronize()
    eager = []
    for label, rows, width, G, dtype, flags, shape, yd, gd, wd, od, ref in cases:
        assert_parity(host_bits(od, dtype), ref, dtype, f"graph job {label}")
        eager.append(od.clone())

    graph = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    with torch.cuda.graph(graph, stream=cs):
        launch_all(cs)
    for rep in range(4):
        say(f"case graph of kernel families: replay {rep}")
        for *_, od, _ in cases:
            od.fill_(0)
        junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert junk.isfinite()
        for (label, *_, od, _), e in zip(cases, eager):
            assert torch.equal(od.view(torch.int16), e.view(torch.int16)), (label, rep)
