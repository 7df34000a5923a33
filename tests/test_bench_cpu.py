"""bench.py's host side on the CPU: the one-GPU guard, the workload it times,
and the CPU baseline leg (the oracle on a bounded sample of that workload,
single-threaded and over the host's cores).  Nothing here needs a GPU."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_more_than_one_gpu_is_refused():
    """Several GPUs exit with status 2 and a reason, before torch is imported
    and without printing a result line."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2, r
    assert "one GPU" in r.stderr and r.stdout == ""


def test_timed_workload_is_the_prefill():
    """The timed step is the 8192 x 7680 bf16 prefill with groups of 960 and
    the intermediate cast; its algorithmic bytes are y, gate and out once
    (2 bytes each) plus the f32 weight once."""
    b = _bench()
    import synthetic as S

    w = S.WORKLOADS[b.PREFILL]
    assert (w.rows, w.width, w.group_size, w.round_intermediate) == (8192, 7680, 960, 1)
    assert w.esize == 2 and w.algorithmic_bytes() == 3 * 8192 * 7680 * 2 + 4 * 7680
    assert b.PEAK_HBM_GBS == 8000.0


def test_cpu_baseline_leg():
    """The oracle leg returns the documented fields, one core for the
    single-threaded figure, and a positive rate for both figures."""
    b = _bench()
    import synthetic as S

    S.build(force=False)
    res = b.cpu_baseline(S, 0.2)
    assert res["unit"] == "GB/s" and res["kind"] == "oracle" and res["cores"] == 1
    assert res["value"] > 0 and res["rows_per_s"] > 0 and "256 of the 8192 rows" in res["sample"]
    allc = res["all_cores"]
    assert allc["kind"] == "oracle x cores" and allc["cores"] >= 1 and allc["value"] > 0


def _torch_from_storage(torch, a, dtype, rows, width):
    import numpy as np

    tdt = {0: torch.float32, 1: torch.float16, 2: torch.bfloat16}[dtype]
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if dtype else a)
    return (t.view(tdt) if dtype else t).reshape(rows, width)


def _bits(torch, t, dtype):
    import numpy as np

    c = t.detach().cpu().reshape(-1)
    return c.numpy() if dtype == 0 else c.view(torch.int16).numpy().view(np.uint16)


def test_unfused_chains_compute_the_op():
    """The PyTorch op chains bench.py times against the fused kernel compute
    the op: run on the CPU over small seeded inputs (bf16 and fp16, the
    intermediate cast on and off, groups of 960 and 128) they meet the parity
    bar against the oracle, gate first and norm first (with a shared scale).

    The 2-ulp bar alone would let a misplaced or missing intermediate cast
    through (it moves an output by at most about one unit), so at least 99%
    of the outputs must also equal the oracle's bit for bit: the chain and
    the oracle differ only in the f32 rounding of the sum, silu and the
    normaliser, which changes an output only when its exact value lies within
    a few f32 ulps of a rounding boundary of the 8- or 11-bit result (measured:
    at least 99.96% equal), whereas taking the other cast point changes about
    a quarter of them (measured: 73-74% equal)."""
    import torch

    import oracle
    import synthetic as S
    from gpu_util import assert_parity

    b = _bench()
    S.build(force=False)
    oracle.build(force=False)
    rows = 16
    for dtype in (S.BF16, S.F16):
        for G, width in ((960, 1920), (128, 1024)):
            y = S.tensor(77, S.TID_Y, rows * width, dtype, ("normal", 2.0))
            gt = S.tensor(77, S.TID_GATE, rows * width, dtype, ("normal", 1.0))
            w = S.tensor(77, S.TID_W, width, S.F32, ("uniform", 0.5, 1.5))
            yt = _torch_from_storage(torch, y, dtype, rows, width)
            gtt = _torch_from_storage(torch, gt, dtype, rows, width)
            for ri in (0, 1):
                got = b.unfused_chain(torch, yt, gtt, torch.from_numpy(w), G, 1e-5, ri)
                ref = oracle.forward(y, gt, w, rows=rows, width=width, group_size=G,
                                     y_row_stride=width, gate_row_stride=width,
                                     out_row_stride=width, eps=1e-5, dtype=dtype,
                                     round_intermediate=ri)
                st = assert_parity(_bits(torch, got, dtype), ref, dtype, f"chain {dtype} G{G} ri{ri}")
                assert st["exact"] >= 0.99, (dtype, G, ri, st)
            wg = w[:G].copy()
            got = b.unfused_chain_norm_first(torch, yt, gtt, torch.from_numpy(wg), G, 1e-6)
            ref = oracle.forward(y, gt, wg, rows=rows, width=width, group_size=G,
                                 y_row_stride=width, gate_row_stride=width, out_row_stride=width,
                                 eps=1e-6, dtype=dtype, norm_before_gate=True,
                                 weight_per_group=True)
            st = assert_parity(_bits(torch, got, dtype), ref, dtype, f"norm-first chain {dtype} G{G}")
            assert st["exact"] >= 0.99, (dtype, G, st)


def test_traffic_figure_follows_the_kernel_sources():
    """The traffic figure is read only while the sources it was measured on
    are unchanged; every source that the hash covers exists."""
    b = _bench()
    for p in b.KERNEL_SOURCES:
        assert os.path.isfile(os.path.join(ROOT, p)), p
    h = b.kernel_source_hash()
    assert len(h) == 16
    fig = b.traffic_figure()
    assert fig is None or fig > 0
