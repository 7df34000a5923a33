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
