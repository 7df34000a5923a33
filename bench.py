"""Benchmark of the fused gated group-RMSNorm on one MI355X.

A step is one launch of the fused kernel over the 8192 x 7680 bf16 prefill
batch (group size 960, intermediate cast on): every stage of the op (widen,
silu gate, group sum of squares, normaliser, optional intermediate cast,
weight multiply, narrow and store) runs inside it.  Inputs are resident in
HBM before timing; several copies of them are rotated so no step finds its
inputs in the 256 MB last-level cache.

Printed (one JSON line): the kernel's achieved HBM throughput in GB/s
(algorithmic bytes over the event-timed average of the timed back-to-back
launches; also the host wall-clock rate and the median single launch,
labelled), the kernel's roofline figures, the
decode latency (1 x 7680, 21 layers back to back issued from C, eager and
graph-replayed, next to an empty kernel of the same grid), the unfused
four-op chain in PyTorch eager, and the CPU oracle timed on a bounded
sample of the same workload.

  python bench.py [--gpus 1] [--steps K] [--warmup W]
                  [--only prefill|decode|copy|workloads|unfused|shapes|evidence]
                  [--part prefill|gdn|decode] [--variant NAME]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (fraction of peak) at 8192x7680 bf16; µs/launch at 1x7680 decode"
PEAK_HBM_GBS = 8000.0
PREFILL = "mamba2_prefill_8192x7680_bf16_g960"
DECODE = "mamba2_decode_1x7680_bf16_g960"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_prefill_8192x7680_bf16.md")
KERNEL_SOURCES = ["gated_group_rmsnorm_amd/csrc/ggrms_kernels.hpp",
                  "gated_group_rmsnorm_amd/csrc/ggrms_epilogue.hpp",
                  "gated_group_rmsnorm_amd/csrc/table_bf16.hip",
                  "gated_group_rmsnorm_amd/csrc/plan.cpp"]


# ggrms_flag_t bits (include/ggrms.h); the others are launch controls
OPERATOR_FLAGS = 1 | 2 | 4


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed launches for this long after the warmup steps")
    ap.add_argument("--only", choices=["prefill", "decode", "copy", "workloads", "unfused",
                                       "shapes", "evidence", "producer"], default=None)
    ap.add_argument("--part", choices=list(UNFUSED_PARTS), default=None,
                    help="with --only unfused: time one chain only")
    ap.add_argument("--variant", choices=sorted(EVIDENCE), default="prefill_staged",
                    help="with --only evidence: the launch-choice job to time")
    ap.add_argument("--decode-bursts", type=int, default=200)
    ap.add_argument("--decode-eager-only", action="store_true",
                    help="with --only decode: eager bursts only, no graph capture")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--shape", default=None,
                    help="force a kernel shape 'lanes,vectors[,rows_per_workgroup]'")
    return ap.parse_args()


class Setup:
    """Device copies of a workload's inputs (several rotating sets) and outputs."""

    def __init__(self, torch, S, w, sets: int, layer: int = 0, flags=None):
        import numpy as np

        self.w = w
        # flags of ggrms_forward_ex/_tuned: the workload's own gate-first
        # rounding unless given; a shared group weight takes the first
        # group_size values of the workload's weight
        self.flags = (1 if w.round_intermediate else 0) if flags is None else flags
        tdt = {S.F32: torch.float32, S.F16: torch.float16, S.BF16: torch.bfloat16}[w.dtype]
        ybuf, gbuf, wt, lay = S.make_inputs(w, layer)
        if self.flags & 4:
            wt = np.ascontiguousarray(wt[:w.group_size])
        self.lay = lay

        def dev(a):
            t = torch.from_numpy(a.view(np.int16) if w.dtype != S.F32 else a)
            return (t.view(tdt) if w.dtype != S.F32 else t).cuda()

        self.weight = torch.from_numpy(wt).cuda()
        base_y = dev(ybuf)
        base_g = base_y if w.fused_width else dev(gbuf)
        self.sets = []
        for i in range(sets):
            yb = base_y if i == 0 else base_y.clone()
            gb = yb if w.fused_width else (base_g if i == 0 else base_g.clone())
            out = torch.empty(w.rows * w.width, dtype=tdt, device="cuda")
            self.sets.append((yb[lay["y_offset"]:], gb[lay["gate_offset"]:], out))
        torch.cuda.synchronize()

    def args(self, i=0):
        w, lay = self.w, self.lay
        y, gt, out = self.sets[i % len(self.sets)]
        return (y.data_ptr(), gt.data_ptr(), self.weight.data_ptr(), out.data_ptr(), w.rows,
                w.width, w.group_size, lay["y_row_stride"], lay["gate_row_stride"], w.width,
                w.eps, w.dtype, self.flags)

    def launch(self, g, i, stream, shape=None):
        # the public entry point, unless a shape or a launch control is forced
        if shape is None and not self.flags & ~OPERATOR_FLAGS:
            st = g.ggrms_forward_ex(*self.args(i), stream)
        else:
            st = g.ggrms_forward_tuned(*self.args(i), stream, shape)
        if st != 0:
            raise RuntimeError(f"ggrms_forward: {g.ggrms_status_string(st)}")

    def plan(self, g, shape=None):
        st, p = g.ggrms_plan_tuned(*self.args(), shape)
        if st != 0:
            raise RuntimeError(f"ggrms_plan_tuned: {g.ggrms_status_string(st)}")
        return p


def settle(torch, launch, seconds):
    """Untimed launches until `seconds` of wall time have passed: from idle the
    GPU needs ~30 ms (~500 launches of the prefill kernel) to reach its
    steady clocks, and a measurement taken inside that ramp reads ~5-10% low."""
    t0 = time.perf_counter()
    i = 0
    while True:
        for _ in range(32):
            launch(i)
            i += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return i


def time_kernel(torch, g, setup, steps, warmup, shape=None, settle_s=0.2):
    """`warmup` untimed launches, then untimed launches for `settle_s`
    seconds, then `steps` back-to-back launches between two HIP events
    recorded on the launch stream, with the host wall clock around them.
    Returns (wall_s, event_ms_total)."""
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    for i in range(warmup):
        setup.launch(g, i, sp, shape)
    settle(torch, lambda i: setup.launch(g, i, sp, shape), settle_s)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        setup.launch(g, i, sp, shape)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, start.elapsed_time(end)


def per_launch_percentiles(torch, g, setup, shape, launches=200):
    """p10 / p50 / p90 of single launches, each between its own pair of HIP
    events on the launch stream (after the timed loop, outside it; the
    rotating input sets keep every launch's inputs out of the caches)."""
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(launches)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        setup.launch(g, i, sp, shape)
        b.record(stream)
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    pick = lambda q: round(us[min(len(us) - 1, int(q * len(us)))], 2)
    return {"p10": pick(0.1), "p50": pick(0.5), "p90": pick(0.9), "launches": launches}


class _OneSet:
    """A Setup whose launches all use input set 0."""

    def __init__(self, setup):
        self.setup = setup

    def launch(self, g, i, stream, shape=None):
        self.setup.launch(g, 0, stream, shape)


def bench_prefill(torch, g, S, args, shape):
    w = S.WORKLOADS[PREFILL]
    nbytes = w.algorithmic_bytes()
    sets = max(2, math.ceil(3 * 256e6 / nbytes))  # > 3x the 256 MB Infinity Cache per rotation
    log(f"prefill: generating {w.name}, {sets} rotating input sets")
    setup = Setup(torch, S, w, sets)
    wall, ev_ms = time_kernel(torch, g, setup, args.steps, args.warmup, shape,
                              args.settle_ms / 1e3)
    plan = setup.plan(g, shape)
    avg_ms = ev_ms / args.steps
    res = {
        "workload": w,
        "bytes": nbytes,
        "wall_s": wall,
        "kernel_ms_avg": avg_ms,
        "setup": setup,
        "per_launch_us": per_launch_percentiles(torch, g, setup, shape),
        "plan": plan,
        "sets": sets,
    }
    log(f"prefill: wall {wall * 1e3 / args.steps:.4f} ms/step, event avg {avg_ms * 1e3:.2f} us "
        f"per launch, {nbytes / (avg_ms * 1e-3) / 1e9:.0f} GB/s")
    return res


def bench_decode(torch, g, S, bursts, eager_only=False):
    """21 back-to-back launches (distinct layer inputs) per burst, issued from
    C through libggrms.so (libggrms_bench.so's loop: no interpreter between
    launches), timed with events around each burst; eager and as one replayed
    HIP graph; next to an empty kernel launched with the same grid the same
    ways; and the graph replayed back to back (the graph's start-up overlapping
    the previous replay).  Also: the same bursts with the streaming cache hint forced (the
    default keeps a job this small cached), and the eager burst issued from
    Python through the ctypes binding, for context."""
    w = S.WORKLOADS[DECODE]
    L = S.DECODE_LAYERS
    layers = [Setup(torch, S, w, 1, layer) for layer in range(L)]
    aux = ctypes.CDLL(os.path.join(ROOT, "gated_group_rmsnorm_amd", "libggrms_bench.so"))
    vp = ctypes.c_void_p
    aux.ggrms_bench_decode_native.argtypes = [
        ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp),
        ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_float, ctypes.c_int,
        ctypes.c_uint32, vp, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double),
        ctypes.POINTER(ctypes.c_double)]
    plan = layers[0].plan(g)
    ptrs = [layers[i].sets[0] for i in range(L)]
    arr = lambda xs: (vp * L)(*xs)
    ys = arr([p[0].data_ptr() for p in ptrs])
    gs = arr([p[1].data_ptr() for p in ptrs])
    ws = arr([ly.weight.data_ptr() for ly in layers])
    outs = arr([p[2].data_ptr() for p in ptrs])

    def native(mode, flags):
        dev, host = ctypes.c_double(), ctypes.c_double()
        rc = aux.ggrms_bench_decode_native(ys, gs, ws, outs, L, w.width, w.group_size, w.eps,
                                           w.dtype, flags, None, bursts, mode,
                                           ctypes.byref(dev), ctypes.byref(host))
        if rc != 0:
            raise RuntimeError(f"ggrms_bench_decode_native mode {mode}: status {rc}")
        return dev.value, host.value

    flags = layers[0].flags
    eager, host = native(0, flags)
    floor_eager, floor_host = native(2, flags)
    if eager_only:  # no graph capture (counter collection runs)
        res = {"workload": w.name, "us_per_launch_eager": eager, "host_us_per_call": host,
               "floor_us_per_launch_eager": floor_eager, "floor_host_us_per_call": floor_host,
               "grid": [plan["workgroups"], plan["block_threads"]]}
        log(f"decode (eager only): {json.dumps(res)}")
        return res
    graph, _ = native(1, flags)
    floor_graph, _ = native(3, flags)
    graph_b2b, _ = native(4, flags)
    floor_graph_b2b, _ = native(5, flags)
    eager_nt, _ = native(0, flags | g.FLAG_CACHE_STREAM)
    graph_nt, _ = native(1, flags | g.FLAG_CACHE_STREAM)

    def python_burst(stream):
        for ly in layers:
            ly.launch(g, 0, stream)

    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    settle(torch, lambda i: python_burst(sp), 0.1)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(bursts)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record(stream)
        python_burst(sp)
        b.record(stream)
    torch.cuda.synchronize()
    py_eager = statistics.median(a.elapsed_time(b) for a, b in evs) * 1e3 / L

    res = {
        "workload": w.name,
        "layers": L,
        "bursts": bursts,
        "cache_policy": "stream" if plan["streaming"] else "keep",
        "us_per_launch_eager": eager,
        "host_us_per_call": host,
        "floor_us_per_launch_eager": floor_eager,
        "floor_host_us_per_call": floor_host,
        "us_per_launch_graph": graph,
        "floor_us_per_launch_graph": floor_graph,
        # the graph replayed back to back (each replay's start overlapping the
        # previous one's tail), per launch; the figure above times each replay
        # alone, its start-up included
        "us_per_launch_graph_back_to_back": graph_b2b,
        "floor_us_per_launch_graph_back_to_back": floor_graph_b2b,
        "us_per_launch_eager_streamed": eager_nt,
        "us_per_launch_graph_streamed": graph_nt,
        "us_per_launch_eager_python": py_eager,
        "grid": [plan["workgroups"], plan["block_threads"]],
    }
    log(f"decode: {json.dumps(res)}")
    return res


def bench_copy(torch, steps):
    """The plain 16-byte copy used to calibrate the traffic counters."""
    aux = ctypes.CDLL(os.path.join(ROOT, "gated_group_rmsnorm_amd", "libggrms_bench.so"))
    aux.ggrms_bench_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                     ctypes.c_void_p]
    nbytes = 256 << 20
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    sp = torch.cuda.current_stream().cuda_stream
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record()
        if aux.ggrms_bench_copy(src.data_ptr(), dst.data_ptr(), nbytes, sp) != 0:
            raise RuntimeError("copy launch failed")
        b.record()
    torch.cuda.synchronize()
    ms = statistics.fmean(a.elapsed_time(b) for a, b in ev)
    log(f"copy: {nbytes} B read + {nbytes} B written per launch, {ms * 1e3:.1f} us, "
        f"{2 * nbytes / (ms * 1e-3) / 1e9:.0f} GB/s")
    return {"bytes_read": nbytes, "bytes_written": nbytes, "kernel_ms_avg": ms}


def stream_ceiling(torch, nbytes, steps, settle_s=0.1, fill="random"):
    """Event-timed average launch of the plain two-read-one-write kernel
    (libggrms_bench.so's ggrms_bench_stream3) over `nbytes` per stream, with
    as many rotating buffer sets as keep the 256 MB Infinity Cache cold, after
    the same warm-up and settle as the fused kernel.  The buffers hold random
    normal f32 values like the fused kernel's inputs (fill="constant": 0.5
    everywhere; the HBM rate depends slightly on the bits moved).  Returns
    microseconds."""
    aux = ctypes.CDLL(os.path.join(ROOT, "gated_group_rmsnorm_amd", "libggrms_bench.so"))
    aux.ggrms_bench_stream3.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int64, ctypes.c_void_p]
    nbytes = (nbytes + 15) // 16 * 16
    sets = min(64, max(2, math.ceil(3 * 256e6 / (3 * nbytes))))
    def buf():
        t = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
        return t.normal_() if fill == "random" else t.fill_(0.5)

    bufs = [[buf() for _ in range(3)] for _ in range(sets)]
    sp = torch.cuda.current_stream().cuda_stream

    def launch(i):
        a, b, c = bufs[i % sets]
        if aux.ggrms_bench_stream3(a.data_ptr(), b.data_ptr(), c.data_ptr(), nbytes, sp) != 0:
            raise RuntimeError("stream3 launch failed")

    for i in range(5):
        launch(i)
    settle(torch, launch, settle_s)
    a_ev = torch.cuda.Event(enable_timing=True)
    b_ev = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a_ev.record()
    for i in range(steps):
        launch(i)
    b_ev.record()
    torch.cuda.synchronize()
    del bufs
    torch.cuda.empty_cache()
    return a_ev.elapsed_time(b_ev) * 1e3 / steps


# (label, workload, ggrms_forward_ex flags or None for the workload's own)
OTHER_WORKLOADS = [
    ("strided_256x4800_f16_g100", "strided_256x4800_f16_g100", None),
    # gate first, the 128-value head scale shared by every head (the page's
    # [C] scale), and the same scale tiled into a per-column weight
    ("gdn_head_16384x8192_f16_g128", "gdn_head_16384x8192_f16_g128", 4),
    ("gdn_head_16384x8192_f16_g128_per_column_weight", "gdn_head_16384x8192_f16_g128", None),
    # norm first with the shared head scale
    ("gdn_head_16384x8192_f16_g128_norm_first", "gdn_head_16384x8192_f16_g128", 2 | 4),
    ("prefill_8192x7680_bf16_g960_norm_first", PREFILL, 2),
]


def native_job_us(setup, kind, launches, bursts=20):
    """Per-launch time of `launches` back-to-back launches issued from C
    (libggrms_bench.so's ggrms_bench_job_native) over the setup's rotating
    buffer sets, median of `bursts` runs: kind 0 the fused kernel (the
    library's own launch choice), kind 1 the plain two-read-one-write kernel
    over the same views (y and gate read, out written; strided rows where the
    views are strided, e.g. column slices of one fused buffer).  Issued from C, a small
    job's figure is the GPU's: from Python each launch costs about 4 us of
    interpreter and ctypes time, as long as the strided workload's kernel."""
    aux = ctypes.CDLL(os.path.join(ROOT, "gated_group_rmsnorm_amd", "libggrms_bench.so"))
    f = aux.ggrms_bench_job_native
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                  ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                  ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_uint32, ctypes.c_void_p,
                  ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    n = len(setup.sets)
    arr = lambda vals: (ctypes.c_void_p * n)(*vals)
    ys = arr([y.data_ptr() for y, _, _ in setup.sets])
    gs = arr([gt.data_ptr() for _, gt, _ in setup.sets])
    os_ = arr([o.data_ptr() for _, _, o in setup.sets])
    w, lay = setup.w, setup.lay
    us = ctypes.c_double()
    rc = f(ys, gs, setup.weight.data_ptr(), os_, n, w.rows, w.width, w.group_size,
           lay["y_row_stride"], lay["gate_row_stride"], w.width, w.eps, w.dtype, setup.flags, None,
           kind, launches, bursts, ctypes.byref(us))
    if rc != 0:
        raise RuntimeError(f"ggrms_bench_job_native kind {kind}: status {rc}")
    return us.value


def bench_workloads(torch, g, S, steps):
    """Kernel time of the other configured workloads and of the norm-first
    operator (reported beside the headline): back-to-back launches issued
    from C, next to the plain stream kernel over the same buffers."""
    out = {}
    for label, name, flags in OTHER_WORKLOADS:
        w = S.WORKLOADS[name]
        sets = max(2, math.ceil(3 * 256e6 / w.algorithmic_bytes()))
        setup = Setup(torch, S, w, min(sets, 64), flags=flags)
        avg = native_job_us(setup, 0, steps) * 1e-3  # ms
        ceil_us = native_job_us(setup, 1, steps)
        nbytes = w.algorithmic_bytes(per_group_weight=bool(setup.flags & 4))
        del setup
        torch.cuda.empty_cache()
        out[label] = {"kernel_us_avg": avg * 1e3,
                      "gbs": nbytes / (avg * 1e-3) / 1e9,
                      "frac_of_peak": nbytes / (avg * 1e-3) / 1e9 / PEAK_HBM_GBS,
                      "rows_per_s": w.rows / (avg * 1e-3),
                      "stream_ceiling_us": ceil_us,
                      "frac_of_stream_ceiling": ceil_us / (avg * 1e3)}
    log(f"workloads: {json.dumps(out)}")
    return out


# Model-shaped jobs at the prefill's size (~125.8 MB per stream): (label,
# dtype, group size, width, ggrms_forward_tuned flags[, row stride]).  Group sizes of Mamba-2
# mixers (d_inner / n_groups for 8 or fewer groups), per-head norms with a
# shared head weight, both operators, the three element types.
SHAPES = [
    ("bf16 G960 gate first (the prefill workload)", 2, 960, 7680, 1),
    ("bf16 G960 norm first", 2, 960, 7680, 2),
    ("fp16 G960 gate first", 1, 960, 7680, 1),
    ("f32 G960 gate first", 0, 960, 7680, 0),
    ("f32 G960 norm first", 0, 960, 7680, 2),
    ("bf16 G1024, 8 groups of a 8192-wide row", 2, 1024, 8192, 1),
    ("bf16 G2048, 8 groups of a 16384-wide row", 2, 2048, 16384, 1),
    ("bf16 G3584, 2 groups of a 7168-wide row", 2, 3584, 7168, 1),
    ("bf16 G5120, one group per row", 2, 5120, 5120, 1),
    ("bf16 G8192, one group per row", 2, 8192, 8192, 1),
    ("bf16 G12288, one group per row", 2, 12288, 12288, 1),
    ("bf16 G16384, one group per row", 2, 16384, 16384, 1),
    ("fp16 G128 heads, per-column weight", 1, 128, 8192, 0),
    ("bf16 G128, 60 groups of a 7680-wide row, per-column weight", 2, 128, 7680, 1),
    ("bf16 G128, 64 groups of a 8192-wide row, per-column weight", 2, 128, 8192, 1),
    ("fp16 G128 heads, shared head weight", 1, 128, 8192, 4),
    ("fp16 G128 heads, norm first, shared head weight", 1, 128, 8192, 6),
    ("fp16 G256 heads, shared head weight", 1, 256, 8192, 4),
    ("f32 G128 heads, shared head weight", 0, 128, 4096, 4),
    ("fp16 G100 packed groups, per-column weight", 1, 100, 4800, 1),
    ("fp16 G100 packed groups, shared head weight", 1, 100, 4800, 1 | 4),
    ("bf16 G99 packed groups (2-byte pieces)", 2, 99, 4752, 1),
    ("bf16 G127 packed groups (runs of 8)", 2, 127, 6096, 1),
    ("bf16 G127 packed groups, shared head weight", 2, 127, 6096, 1 | 4),
    ("fp16 G13 packed groups (runs of 32)", 1, 13, 4992, 1),
    ("fp16 G250 packed groups (4-byte pieces)", 1, 250, 12000, 1),
    # the same groups in rows padded by 4 elements: rows not 16-byte aligned,
    # so the whole group falls back to 8-byte vectors
    ("fp16 G100 in padded rows (8-byte vectors)", 1, 100, 4800, 1, 4804),
]


def bench_shapes(torch, g, steps):
    """The fused kernel on model-shaped jobs of ~377 MB (three streams of
    125,829,120 B each, three rotating sets, random normal inputs), each next
    to the plain two-read-one-write kernel moving the same bytes."""
    tb = 125829120
    sets = 3
    raw = [[torch.empty(tb, dtype=torch.uint8, device="cuda") for _ in range(3)] for _ in range(sets)]
    weight = torch.rand(16384, device="cuda") + 0.5
    sp = torch.cuda.current_stream().cuda_stream
    tdt = {0: torch.float32, 1: torch.float16, 2: torch.bfloat16}
    ceil_us = stream_ceiling(torch, tb, steps)
    const_us = stream_ceiling(torch, tb, steps, fill="constant")
    log(f"plain two-read-one-write kernel at 3 x {tb} B: {ceil_us:.2f} us on random data, "
        f"{const_us:.2f} us on constant data")
    out = {"stream_ceiling_us": ceil_us, "stream_ceiling_constant_data_us": const_us,
           "shapes": []}
    for label, dt, G, width, flags, *pad in SHAPES:
        esz = 4 if dt == 0 else 2
        stride = pad[0] if pad else width
        rows = tb // esz // stride
        views = []
        for y, gt, o in raw:
            yv, gv = y.view(tdt[dt]), gt.view(tdt[dt])
            yv.normal_()
            gv.normal_()
            views.append((yv, gv, o.view(tdt[dt])))

        def launch(i):
            y, gt, o = views[i % sets]
            st = g.ggrms_forward_tuned(y.data_ptr(), gt.data_ptr(), weight.data_ptr(), o.data_ptr(),
                                    rows, width, G, stride, stride, stride, 1e-5, dt, flags, sp)
            if st != 0:
                raise RuntimeError(f"{label}: {g.ggrms_status_string(st)}")

        for i in range(5):
            launch(i)
        settle(torch, launch, 0.1)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for i in range(steps):
            launch(i)
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / steps
        nbytes = 3 * rows * width * esz
        st, p = g.ggrms_plan_tuned(views[0][0].data_ptr(), views[0][1].data_ptr(), weight.data_ptr(),
                                views[0][2].data_ptr(), rows, width, G, stride, stride, stride,
                                1e-5, dt, flags)
        rec = {"label": label, "rows": rows, "width": width, "row_stride": stride,
               "group_size": G, "flags": flags,
               "us": round(us, 2), "frac_of_peak": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
               "frac_of_stream_ceiling": round(ceil_us * nbytes / (3 * tb) / us, 4),
               "shape": f"{p['kernel_name']} {p['lanes_per_group']}x{p['vectors_per_lane']} "
                        f"rows/wg {p['rows_per_workgroup']} vector {p['vector_bytes']} B"
                        f" piece {p['piece_bytes']} B"}
        out["shapes"].append(rec)
        log(f"{label:50s} {rec['shape']:40s} {us:8.2f} us {rec['frac_of_peak']:.3f} of peak "
            f"{rec['frac_of_stream_ceiling']:.3f} of the plain stream")
    del raw
    torch.cuda.empty_cache()
    return out


# Launch-choice A/B jobs whose counters back the design (each ~377 MB, three
# rotating sets of random inputs): (dtype, rows, width, group size, flags of
# ggrms_forward_tuned, forced shape or None).  The prefill with its weights
# staged in LDS (4 rows of a group per workgroup, the default) and with one
# row per workgroup (each unit reads its own weights); 9 groups of 960 per
# row, where the row-major order makes every XCD read every group's weights,
# in the XCD-banded order (the default) and in row-major order; the
# single-group rows of Mamba-2 mixers with one group (G = 5120, 8192), with
# workgroups taking rows in turn (ROWS, the default) and one row per
# workgroup (BLOCK); and packed groups.
EVIDENCE = {
    "prefill_staged": (2, 8192, 7680, 960, 1, None),
    "prefill_unstaged": (2, 8192, 7680, 960, 1, (128, 1, 1)),
    "g9_banded": (2, 7281, 8640, 960, 1 | 64, None),
    "g9_rows": (2, 7281, 8640, 960, 1 | 32, None),
    # WAVE shapes whose row is not a whole number of 8 workgroups: 60 groups of
    # 128 (15 one-wave workgroups of 4 groups per row) and 12 groups of 640
    # (64 x 2, one wave per group), banded and row-major
    "g128x60_banded": (2, 8192, 7680, 128, 1 | 64, None),
    "g128x60_rows": (2, 8192, 7680, 128, 1 | 32, None),
    "g640x12_banded": (2, 8192, 7680, 640, 1 | 64, None),
    "g640x12_rows": (2, 8192, 7680, 640, 1 | 32, None),
    "g5120": (2, 12288, 5120, 5120, 1, None),
    "g5120_block": (2, 12288, 5120, 5120, 1, (256, 3, 1)),
    "g8192": (2, 7680, 8192, 8192, 1, None),
    "g8192_block": (2, 7680, 8192, 8192, 1, (256, 4, 1)),
    # one group of 12288 per row: ROWS 768 x 2 (the default) and BLOCK 256 x 6;
    # one group of 16384: BLOCK 512 x 4 (the default) and ROWS 1024 x 2
    "g12288": (2, 5120, 12288, 12288, 1, None),
    "g12288_block": (2, 5120, 12288, 12288, 1, (256, 6, 1)),
    "g16384": (2, 3840, 16384, 16384, 1, None),
    "g16384_rows": (2, 3840, 16384, 16384, 1, (1024, 2, 0, 0, 5)),
    # 100-wide fp16 groups (200 bytes: packed 16-byte vectors), one vector per
    # lane on 16 lanes (the library's shape) and two vectors per lane on 8
    # lanes (boundary vectors in pieces)
    "packed_g100": (1, 13107, 4800, 100, 1, None),
    "packed_g100_8x2": (1, 13107, 4800, 100, 1, (8, 2)),
    # the same groups in runs of 5 per wave (one vector per lane) and of 10
    # (two vectors per lane, every run on a vector boundary)
    "packed_g100_run": (1, 13107, 4800, 100, 1, (64, 1, 0, 0, 4)),
    "packed_g100_run2": (1, 13107, 4800, 100, 1, (64, 2, 0, 0, 4)),
    # 16 x 1 in four-wave workgroups (16 groups = 3200 bytes, whole 128-byte
    # lines, per workgroup), and both workgroup sizes in row-major order
    "packed_g100_four": (1, 13107, 4800, 100, 1 | 256, None),
    "packed_g100_rows": (1, 13107, 4800, 100, 1 | 32, None),
    "packed_g100_rows_four": (1, 13107, 4800, 100, 1 | 32 | 256, None),
    # 127-wide bf16 groups (15.9 vectors on 32 lanes): runs of 8 on two vectors
    # per lane (the default) and the 32-lane segments
    "packed_g127_run": (2, 10320, 6096, 127, 1, None),
    "packed_g127_wave": (2, 10320, 6096, 127, 1, (32, 1)),
    # groups that nearly fill 32-lane segments (the library's choice) against
    # runs of groups on two vectors per lane: 250-wide fp16 (31.3 vectors),
    # 230-wide bf16 (28.8), 180-wide bf16 (22.5)
    "packed_g250": (1, 5242, 12000, 250, 1, None),
    "packed_g250_run2": (1, 5242, 12000, 250, 1, (64, 2, 0, 0, 4)),
    "packed_g230": (2, 8548, 7360, 230, 1, None),
    "packed_g230_run2": (2, 8548, 7360, 230, 1, (64, 2, 0, 0, 4)),
    "packed_g180": (2, 7281, 8640, 180, 1, None),
    "packed_g180_run2": (2, 7281, 8640, 180, 1, (64, 2, 0, 0, 4)),
    # more groups on 32-lane segments with 4-byte pieces: 222-wide bf16 (27.8
    # vectors), 210-wide fp16 (26.3), 170-wide bf16 (21.3), 99-wide f32 (24.8)
    "packed_g222": (2, 8856, 7104, 222, 1, None),
    "packed_g222_run2": (2, 8856, 7104, 222, 1, (64, 2, 0, 0, 4)),
    "packed_g210": (1, 8322, 7560, 210, 1, None),
    "packed_g210_run2": (1, 8322, 7560, 210, 1, (64, 2, 0, 0, 4)),
    "packed_g170": (2, 8411, 7480, 170, 1, None),
    "packed_g170_run2": (2, 8411, 7480, 170, 1, (64, 2, 0, 0, 4)),
    "packed_g99f32": (0, 4180, 7524, 99, 0, None),
    "packed_g99f32_run2": (0, 4180, 7524, 99, 0, (64, 2, 0, 0, 4)),
}


def bench_evidence(torch, g, variant, steps, warmup, settle_s):
    """Event-timed average launch of one EVIDENCE job (for counter runs:
    `rocprofv3 --pmc ... -- python3 bench.py --only evidence --variant X`)."""
    dt, rows, width, G, flags, shape = EVIDENCE[variant]
    esz = 4 if dt == 0 else 2
    tdt = {0: torch.float32, 1: torch.float16, 2: torch.bfloat16}[dt]
    sets = [[torch.randn(rows * width, device="cuda").to(tdt) for _ in range(2)] +
            [torch.empty(rows * width, dtype=tdt, device="cuda")] for _ in range(3)]
    weight = torch.rand(width, device="cuda") + 0.5
    sp = torch.cuda.current_stream().cuda_stream

    def launch(i):
        y, gt, o = sets[i % 3]
        st = g.ggrms_forward_tuned(y.data_ptr(), gt.data_ptr(), weight.data_ptr(), o.data_ptr(),
                                   rows, width, G, width, width, width, 1e-5, dt, flags, sp, shape)
        if st != 0:
            raise RuntimeError(f"{variant}: {g.ggrms_status_string(st)}")

    for i in range(warmup):
        launch(i)
    if settle_s > 0:
        settle(torch, launch, settle_s)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for i in range(steps):
        launch(i)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / steps
    _, p = g.ggrms_plan_tuned(sets[0][0].data_ptr(), sets[0][1].data_ptr(), weight.data_ptr(),
                              sets[0][2].data_ptr(), rows, width, G, width, width, width, 1e-5,
                              dt, flags, shape)
    nbytes = 3 * rows * width * esz + 4 * width
    rec = {"variant": variant, "rows": rows, "width": width, "group_size": G, "flags": flags,
           "us": round(us, 2), "frac_of_peak": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
           "plan": {k: p[k] for k in ("kernel_name", "lanes_per_group", "vectors_per_lane",
                                      "rows_per_workgroup", "block_threads", "workgroups",
                                      "tile_order", "vector_bytes")}}
    print(json.dumps(rec), flush=True)
    return rec


def unfused_chain(torch, y, gate, w, group_size, eps, ri):
    """The four-op chain the fused kernel replaces, in PyTorch eager: widen,
    silu(gate) * y, group RMSNorm (torch's rms_norm over groups), weight
    multiply and narrow (with the intermediate cast when ri is set)."""
    rows, width = y.shape
    a = torch.nn.functional.silu(gate.float()) * y.float()
    t = torch.nn.functional.rms_norm(a.view(rows, width // group_size, group_size),
                                     (group_size,), eps=eps).view(rows, width)
    if ri:
        t = t.to(y.dtype).float()
    return (w * t).to(y.dtype)


def unfused_chain_norm_first(torch, y, gate, w, group_size, eps):
    """The norm-first operator as PyTorch eager ops: rms_norm over groups of
    the widened y, times the shared group weight, times silu(gate), narrow."""
    rows, width = y.shape
    t = torch.nn.functional.rms_norm(y.float().view(rows, width // group_size, group_size),
                                     (group_size,), eps=eps)
    t = (t * w).view(rows, width) * torch.nn.functional.silu(gate.float())
    return t.to(y.dtype)


UNFUSED_PARTS = ("prefill", "gdn", "decode")


def bench_unfused(torch, S, steps, parts=UNFUSED_PARTS, settle_s=0.2):
    """Per-launch time of the unfused chain beside the fused kernel: the
    prefill batch (eager, back to back), the norm-first chain on the
    16384x8192 fp16 GDN-shaped batch, and the 21-layer decode burst (eager
    and as one replayed graph); `parts` picks which (a kernel trace of one
    part counts that chain's dispatches per pass)."""
    import numpy as np

    res = {}
    if "prefill" in parts:
        res.update(_unfused_prefill(torch, S, steps, settle_s))
    if "gdn" in parts:
        res.update(_unfused_gdn(torch, S, steps, settle_s))
    if "decode" in parts:
        res.update(_unfused_decode(torch, S, settle_s))
    log(f"unfused chain: {json.dumps(res)}")
    return res


def _unfused_prefill(torch, S, steps, settle_s):
    import numpy as np

    res = {}
    w = S.WORKLOADS[PREFILL]
    yb, gb, wt, _ = S.make_inputs(w)
    y = torch.from_numpy(yb.view(np.int16)).view(torch.bfloat16).reshape(w.rows, w.width).cuda()
    gt = torch.from_numpy(gb.view(np.int16)).view(torch.bfloat16).reshape(w.rows, w.width).cuda()
    wd = torch.from_numpy(wt).cuda()
    run = lambda i: unfused_chain(torch, y, gt, wd, w.group_size, w.eps, w.round_intermediate)
    settle(torch, run, settle_s)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        run(i)
    b.record()
    torch.cuda.synchronize()
    res["prefill_us"] = a.elapsed_time(b) * 1e3 / steps
    del y, gt
    torch.cuda.empty_cache()
    return res


def _unfused_gdn(torch, S, steps, settle_s):
    import numpy as np

    res = {}
    n = S.WORKLOADS["gdn_head_16384x8192_f16_g128"]
    yb, gb, wt, _ = S.make_inputs(n)
    y = torch.from_numpy(yb.view(np.int16)).view(torch.float16).reshape(n.rows, n.width).cuda()
    gt = torch.from_numpy(gb.view(np.int16)).view(torch.float16).reshape(n.rows, n.width).cuda()
    wd = torch.from_numpy(np.ascontiguousarray(wt[:n.group_size])).cuda()
    run = lambda i: unfused_chain_norm_first(torch, y, gt, wd, n.group_size, n.eps)
    settle(torch, run, settle_s)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        run(i)
    b.record()
    torch.cuda.synchronize()
    res["gdn_norm_first_us"] = a.elapsed_time(b) * 1e3 / steps
    del y, gt
    torch.cuda.empty_cache()
    return res


def _unfused_decode(torch, S, settle_s):
    import numpy as np

    res = {}
    d = S.WORKLOADS[DECODE]
    layers = []
    for layer in range(S.DECODE_LAYERS):
        yb, gb, wt, _ = S.make_inputs(d, layer)
        layers.append((torch.from_numpy(yb.view(np.int16)).view(torch.bfloat16).reshape(1, d.width).cuda(),
                       torch.from_numpy(gb.view(np.int16)).view(torch.bfloat16).reshape(1, d.width).cuda(),
                       torch.from_numpy(wt).cuda()))

    def burst(i=0):
        for ly, lg, lw in layers:
            unfused_chain(torch, ly, lg, lw, d.group_size, d.eps, d.round_intermediate)

    settle(torch, burst, settle_s / 2)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(100)]
    for x, z in evs:
        x.record()
        burst()
        z.record()
    torch.cuda.synchronize()
    res["decode_us_per_layer_eager"] = statistics.median(x.elapsed_time(z) for x, z in evs) * 1e3 / len(layers)
    cs = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cs):
        burst()
    settle(torch, lambda i: graph.replay(), settle_s / 2)
    for x, z in evs:
        x.record()
        graph.replay()
        z.record()
    torch.cuda.synchronize()
    res["decode_us_per_layer_graph"] = statistics.median(x.elapsed_time(z) for x, z in evs) * 1e3 / len(layers)
    return res


def bench_producer(torch, steps, settle_s=0.2):
    """The epilogue called from a producer kernel (libggrms_example.so: y =
    bf16(x @ wt^T) on the matrix cores, normalised in the same kernel) against
    the same producer storing y followed by the library's launch on it, on the
    8192 x 7680 bf16 prefill shape with groups of 960 and K = 64; three rotating
    sets of gate, y and out.  Random bf16 x and wt: timing only (the example's
    results are checked by tests/test_gpu_example_producer.py)."""
    import ctypes

    import gated_group_rmsnorm_amd as g

    lib = ctypes.CDLL(os.path.join(os.path.dirname(os.path.abspath(g.__file__)),
                                   "libggrms_example.so"))
    ex = lib.ggrms_example_gemm_norm
    ex.restype = ctypes.c_int
    ex.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 4 + [ctypes.c_float, ctypes.c_int,
                                                                   ctypes.c_int, ctypes.c_void_p]
    rows, width, G, K = 8192, 7680, 960, 64
    bf = torch.bfloat16
    x = (torch.randn(rows * K, device="cuda") * 0.1).to(bf)
    wt = (torch.randn(width * K, device="cuda") * 0.1).to(bf)
    w = torch.rand(width, device="cuda") + 0.5
    sets = [[torch.randn(rows * width, device="cuda").to(bf), torch.empty(rows * width, dtype=bf, device="cuda"),
             torch.empty(rows * width, dtype=bf, device="cuda")] for _ in range(3)]
    sp = torch.cuda.current_stream().cuda_stream

    def fused(i):
        gt, _, o = sets[i % 3]
        if ex(x.data_ptr(), wt.data_ptr(), gt.data_ptr(), w.data_ptr(), o.data_ptr(), rows, width,
              K, G, 1e-5, 1, 0, sp) != 0:
            raise RuntimeError("example producer refused its arguments")

    def produce(i):
        gt, y, _ = sets[i % 3]
        if ex(x.data_ptr(), wt.data_ptr(), gt.data_ptr(), w.data_ptr(), y.data_ptr(), rows, width,
              K, G, 1e-5, 1, 1, sp) != 0:
            raise RuntimeError("example producer refused its arguments")

    def norm(i):
        gt, y, o = sets[i % 3]
        st = g.ggrms_forward_ex(y.data_ptr(), gt.data_ptr(), w.data_ptr(), o.data_ptr(), rows,
                                width, G, width, width, width, 1e-5, 2, 1, sp)
        if st != 0:
            raise RuntimeError(g.ggrms_status_string(st))

    def unfused(i):
        produce(i)
        norm(i)

    res = {}
    for name, fn in (("fused_us", fused), ("producer_alone_us", produce), ("norm_alone_us", norm),
                     ("producer_then_norm_us", unfused)):
        settle(torch, fn, settle_s)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for i in range(steps):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        res[name] = a.elapsed_time(b) * 1e3 / steps
    e = rows * width
    res["fused_bytes"] = 2 * (rows * K + width * K) + 2 * e * 2 + 4 * width
    res["unfused_bytes"] = 2 * (rows * K + width * K) + 2 * e + 3 * 2 * e + 4 * width
    res["launches_fused"], res["launches_unfused"] = 1, 2
    return res


def cpu_baseline(S, seconds):
    """The oracle, single-threaded, on leading rows of the prefill workload,
    repeated for about `seconds` of CPU time."""
    import numpy as np

    import oracle

    w = S.WORKLOADS[PREFILL]
    rows = 256
    y, gt = S.make_rows(w, np.arange(rows))
    wt = S.make_weight(w)
    y, gt = y.reshape(-1), gt.reshape(-1)
    sample_bytes = 3 * rows * w.width * w.esize + 4 * w.width
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.forward(y, gt, wt, rows=rows, width=w.width, group_size=w.group_size,
                       y_row_stride=w.width, gate_row_stride=w.width, out_row_stride=w.width,
                       eps=w.eps, dtype=w.dtype, round_intermediate=w.round_intermediate)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    gbs = reps * sample_bytes / el / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{rows} of the 8192 rows of {w.name}, {reps} passes in {el:.1f} s "
                      f"(single-threaded C, one host core)",
            "rows_per_s": round(reps * rows / el, 1),
            "all_cores": cpu_baseline_all_cores(S, y, gt, wt, rows, max(2.0, seconds / 3))}


def cpu_baseline_all_cores(S, y, gt, wt, rows, seconds):
    """The same oracle function on the same rows, the rows split across all
    the host cores this process may use (one thread each; the C call runs
    without the interpreter lock), repeated for about `seconds`."""
    import concurrent.futures as cf

    import numpy as np

    import oracle

    w = S.WORKLOADS[PREFILL]
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    cores = max(1, min(cores, rows))
    bounds = np.linspace(0, rows, cores + 1).astype(int)
    y2, g2 = y.reshape(rows, w.width), gt.reshape(rows, w.width)

    def part(i):
        r0, r1 = bounds[i], bounds[i + 1]
        oracle.forward(np.ascontiguousarray(y2[r0:r1]).reshape(-1),
                       np.ascontiguousarray(g2[r0:r1]).reshape(-1), wt, rows=r1 - r0,
                       width=w.width, group_size=w.group_size, y_row_stride=w.width,
                       gate_row_stride=w.width, out_row_stride=w.width, eps=w.eps,
                       dtype=w.dtype, round_intermediate=w.round_intermediate)

    sample_bytes = 3 * rows * w.width * w.esize + 4 * w.width
    reps = 0
    with cf.ThreadPoolExecutor(cores) as ex:
        t0 = time.perf_counter()
        while True:
            list(ex.map(part, range(cores)))
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    return {"value": round(reps * sample_bytes / el / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle x cores",
            "sample": f"the same {rows} rows split over {cores} threads, {reps} passes in "
                      f"{el:.1f} s"}


def traffic_figure():
    """HBM bytes per launch from the rocprofv3 FETCH_SIZE / WRITE_SIZE runs
    (scaled by the copy-kernel calibration) recorded in the profile summary;
    None if the kernel sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
        current = kernel_source_hash()
    except OSError:
        return None
    fields = dict(line.split(":", 1) for line in text.splitlines()
                  if line.startswith(("hbm_bytes_per_launch:", "kernel_source_hash:")))
    if fields.get("kernel_source_hash", "").strip() != current:
        return None
    try:
        return int(fields["hbm_bytes_per_launch"].strip())
    except (KeyError, ValueError):
        return None


def run_environment(torch, w) -> dict:
    """Where and with what the line was measured: device, runtime, host."""
    props = torch.cuda.get_device_properties(0)
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    cpu_model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"device": props.name, "arch": getattr(props, "gcnArchName", ""),
            "compute_units": props.multi_processor_count,
            "hip": torch.version.hip, "torch": torch.__version__,
            "host_cpu": cpu_model, "host_cores": os.cpu_count(),
            "seed": w.seed, "library_abi": g_abi_version()}


def g_abi_version() -> int:
    import gated_group_rmsnorm_amd as g

    return g.ggrms_abi_version()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported: the fused "
              "norm has no cross-GPU step -- every (row, group) unit is independent, so rows or "
              "whole groups shard across GPUs with no communication.", file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    import gated_group_rmsnorm_amd as g
    import synthetic as S

    S.build(force=False)
    shape = tuple(int(v) for v in args.shape.split(",")) if args.shape else None

    if args.only == "copy":
        bench_copy(torch, args.steps)
        return
    if args.only == "decode":
        bench_decode(torch, g, S, args.decode_bursts, args.decode_eager_only)
        return
    if args.only == "workloads":
        bench_workloads(torch, g, S, args.steps)
        return
    if args.only == "unfused":
        bench_unfused(torch, S, min(args.steps, 100),
                      (args.part,) if args.part else UNFUSED_PARTS, args.settle_ms / 1e3)
        return
    if args.only == "evidence":
        bench_evidence(torch, g, args.variant, min(args.steps, 200), args.warmup,
                       args.settle_ms / 1e3)
        return
    if args.only == "producer":
        res = bench_producer(torch, args.steps, args.settle_ms / 1e3)
        log("producer example: " + json.dumps({k: (round(v, 2) if isinstance(v, float) else v)
                                               for k, v in res.items()}))
        print(json.dumps({"producer_fusion_example": res}), flush=True)
        return
    if args.only == "shapes":
        print(json.dumps(bench_shapes(torch, g, min(args.steps, 300))), flush=True)
        return

    pre = bench_prefill(torch, g, S, args, shape)
    if args.only == "prefill":
        return
    w = pre["workload"]
    # warm: every launch on the same input set, which the 256 MB Infinity
    # Cache then partly holds (reported apart; the headline rate is cold; not
    # part of the --only prefill run that the kernel trace covers)
    _, warm_ms = time_kernel(torch, g, _OneSet(pre["setup"]), args.steps, args.warmup, shape,
                             args.settle_ms / 1e3)
    log(f"prefill, one input set reused: {warm_ms * 1e3 / args.steps:.2f} us per launch")
    del pre["setup"]  # release the prefill's input sets before the other workloads
    ceil_us = stream_ceiling(torch, w.rows * w.width * w.esize, args.steps, args.settle_ms / 1e3)
    log(f"stream ceiling at the prefill's bytes: {ceil_us:.2f} us per launch")
    decode = bench_decode(torch, g, S, args.decode_bursts)
    others = bench_workloads(torch, g, S, max(20, args.steps // 4))
    unfused = bench_unfused(torch, S, 100)
    cpu = None if args.no_cpu_baseline else cpu_baseline(S, args.cpu_seconds)

    nbytes = pre["bytes"]
    # The metric is the kernel's achieved HBM rate: algorithmic bytes over the
    # event-timed average launch (the same figure as roofline.achieved).  The
    # host wall clock around the same launches also holds Python's enqueue
    # and the final synchronisation; it is reported apart, as wall_gbs.
    achieved = nbytes / (pre["kernel_ms_avg"] * 1e-3) / 1e9
    wall_gbs = args.steps * nbytes / pre["wall_s"] / 1e9
    p50 = pre["per_launch_us"]["p50"]
    line = {
        "metric": METRIC,
        "value": round(achieved, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["wall_s"] * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded counter-based N(0, sigma=2) y and gate, U(0.5,1.5) f32 weight",
        "frac_of_peak": round(achieved / PEAK_HBM_GBS, 4),
        # host wall clock around the timed launches (enqueue and sync included)
        "wall_gbs": round(wall_gbs, 1),
        # single launches, each between its own pair of events: median
        "single_launch_p50": {"us": p50, "gbs": round(nbytes / (p50 * 1e-6) / 1e9, 1),
                              "frac": round(nbytes / (p50 * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)},
        "config": {"workload": w.name, "rows": w.rows, "width": w.width,
                   "group_size": w.group_size, "eps": w.eps,
                   "round_intermediate": w.round_intermediate,
                   "rotating_input_sets": pre["sets"], "settle_ms": args.settle_ms,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic_figure(),
                     "algorithmic_bytes_per_launch": nbytes,
                     "kernel_us_avg": round(pre["kernel_ms_avg"] * 1e3, 2),
                     # single launches, each between its own events
                     "kernel_us_per_launch": pre["per_launch_us"],
                     # the plain two-read-one-write kernel moving the same three streams
                     "stream_ceiling_us": round(ceil_us, 2),
                     "stream_ceiling_frac": round(3 * w.rows * w.width * w.esize / (ceil_us * 1e-6)
                                                  / 1e9 / PEAK_HBM_GBS, 4),
                     "frac_of_stream_ceiling": round(ceil_us / (pre["kernel_ms_avg"] * 1e3), 4),
                     # the same launch with one input set reused (partly cached): not the rate
                     "warm_one_input_set_us": round(warm_ms * 1e3 / args.steps, 2)},
        "cpu_baseline": cpu,
        "decode": {k: (round(v, 3) if isinstance(v, float) else v) for k, v in decode.items()},
        "other_workloads": {k: {kk: round(vv, 3) for kk, vv in v.items()} for k, v in others.items()},
        "unfused_chain_torch_eager": {k: round(v, 3) for k, v in unfused.items()},
        "kernel": pre["plan"],
        "env": run_environment(torch, w),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
