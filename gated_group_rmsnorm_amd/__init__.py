"""Fused gated group-RMSNorm for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libggrms.so`` (C ABI in ``include/ggrms.h``;
launch controls for tuning in ``include/ggrms_tuning.h``).  Every step of
the computation runs in the library's HIP kernels; this module only marshals
arguments (and widens a 16-bit weight exactly to the f32 the library
takes).  PyTorch supplies device memory and the
current stream.  There is no fallback: if the library is missing, importing
the binding raises.

The operation, per row n and group g of ``group_size`` contiguous columns
(page "gated_group_rmsnorm", math block)::

    gated = f32(y) * silu(f32(gate))
    nf    = rsqrt(sum(gated^2) / group_size + eps)
    out   = cast(f32(w) * f32(cast(gated * nf, dtype)), dtype)   # round_intermediate
    out   = cast(f32(w) * (gated * nf), dtype)                   # otherwise

and, with FLAG_NORM_BEFORE_GATE, the operator of the page
"com.microsoft.GatedRMSNorm" (Description section), nf taken from y alone::

    out   = cast(((f32(y) * nf) * f32(w)) * silu(f32(gate)), dtype)

The weight has one value per column, or (FLAG_WEIGHT_PER_GROUP) group_size
values shared by every group.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "F32", "F16", "BF16", "FLAG_ROUND_INTERMEDIATE", "FLAG_NORM_BEFORE_GATE",
    "FLAG_WEIGHT_PER_GROUP", "FLAG_CACHE_STREAM", "FLAG_CACHE_KEEP", "FLAG_ORDER_ROWS",
    "FLAG_ORDER_BANDED", "FLAG_WAVE_ONE", "FLAG_WAVE_FOUR", "STREAM_MIN_BYTES", "SUCCESS",
    "ERROR_INVALID_VALUE", "ERROR_NOT_SUPPORTED", "ERROR_LAUNCH", "KERNEL_NAMES", "KERNEL_RUN",
    "KERNEL_ROWS",
    "GgrmsError",
    "ggrms_forward", "ggrms_forward_ex", "ggrms_forward_tuned", "ggrms_plan", "ggrms_plan_ex",
    "ggrms_plan_tuned", "ggrms_status_string", "ggrms_abi_version", "forward", "plan",
    "expand_head_scale", "library_path",
]

F32, F16, BF16 = 0, 1, 2
# operator flags (include/ggrms.h)
FLAG_ROUND_INTERMEDIATE, FLAG_NORM_BEFORE_GATE, FLAG_WEIGHT_PER_GROUP = 1, 2, 4
# launch controls (include/ggrms_tuning.h; the _tuned calls only): cache policy, tile
# order, WAVE workgroup size.  Results are identical whatever they select.
FLAG_CACHE_STREAM, FLAG_CACHE_KEEP = 8, 16
FLAG_ORDER_ROWS, FLAG_ORDER_BANDED, FLAG_WAVE_ONE, FLAG_WAVE_FOUR = 32, 64, 128, 256
STREAM_MIN_BYTES = 4 << 20  # default policy: jobs of at least this many y+gate+out bytes stream
SUCCESS, ERROR_INVALID_VALUE, ERROR_NOT_SUPPORTED, ERROR_LAUNCH = 0, 1, 2, 3
KERNEL_NAMES = {0: "none", 1: "wave", 2: "block", 3: "wide", 4: "run", 5: "rows"}
KERNEL_RUN, KERNEL_ROWS = 4, 5
ABI_VERSION = 5

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libggrms.so")


def library_path() -> str:
    return _LIB_PATH


class GgrmsError(RuntimeError):
    def __init__(self, status: int, what: str = "ggrms_forward"):
        self.status = status
        super().__init__(f"{what}: {ggrms_status_string(status)} (status {status})")


class _Shape(ctypes.Structure):
    _fields_ = [("lanes_per_group", ctypes.c_int32), ("vectors_per_lane", ctypes.c_int32),
                ("rows_per_workgroup", ctypes.c_int32), ("vector_bytes", ctypes.c_int32),
                ("kernel", ctypes.c_int32)]


class _Plan(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("vector_bytes", ctypes.c_int32),
                ("lanes_per_group", ctypes.c_int32), ("vectors_per_lane", ctypes.c_int32),
                ("block_threads", ctypes.c_int32), ("launches", ctypes.c_int32),
                ("rows_per_workgroup", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
                ("workgroups", ctypes.c_int64), ("streaming", ctypes.c_int32),
                ("piece_bytes", ctypes.c_int32), ("tile_order", ctypes.c_int32),
                ("groups_per_run", ctypes.c_int32), ("super_tile", ctypes.c_int32)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it with `python -m gated_group_rmsnorm_amd._build` "
            "(or __graft_entry__.build()); there is no non-HIP fallback")
    L = ctypes.CDLL(_LIB_PATH)
    vp, i64, f32, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    fwd = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, f32, i32, i32]
    L.ggrms_forward.argtypes = fwd + [vp]
    L.ggrms_forward.restype = i32
    L.ggrms_plan.argtypes = fwd + [ctypes.POINTER(_Plan)]
    L.ggrms_plan.restype = i32
    fwd_ex = fwd[:-1] + [ctypes.c_uint32]
    L.ggrms_forward_ex.argtypes = fwd_ex + [vp]
    L.ggrms_forward_ex.restype = i32
    L.ggrms_plan_ex.argtypes = fwd_ex + [ctypes.POINTER(_Plan)]
    L.ggrms_plan_ex.restype = i32
    fwd_tuned = fwd_ex + [ctypes.POINTER(_Shape)]
    L.ggrms_forward_tuned.argtypes = fwd_tuned + [vp]
    L.ggrms_forward_tuned.restype = i32
    L.ggrms_plan_tuned.argtypes = fwd_tuned + [ctypes.POINTER(_Plan)]
    L.ggrms_plan_tuned.restype = i32
    L.ggrms_status_string.argtypes = [i32]
    L.ggrms_status_string.restype = ctypes.c_char_p
    L.ggrms_abi_version.argtypes = []
    L.ggrms_abi_version.restype = i32
    if L.ggrms_abi_version() != ABI_VERSION:
        raise ImportError(f"{_LIB_PATH} has ABI version {L.ggrms_abi_version()}, this binding "
                          f"expects {ABI_VERSION}: rebuild the library")
    return L


_lib = _load()


# ----------------------------------------------------------- raw C calls

def ggrms_forward(y: int, gate: int, norm_weight: int, out: int, rows: int, width: int,
                  group_size: int, y_row_stride: int, gate_row_stride: int,
                  out_row_stride: int, eps: float, dtype: int, round_intermediate: int,
                  stream: int) -> int:
    """The C entry point with device pointers as integers; returns the status."""
    return _lib.ggrms_forward(y, gate, norm_weight, out, rows, width, group_size,
                              y_row_stride, gate_row_stride, out_row_stride, eps, dtype,
                              round_intermediate, stream)


def _shape_arg(shape):
    """None, or (lanes, vectors[, rows per workgroup[, vector bytes[, kernel]]]) as a
    ggrms_shape_t (kernel: 0, KERNEL_RUN for runs of packed groups, or KERNEL_ROWS for
    workgroups that take rows in turn)."""
    if shape is None:
        return None
    f = list(shape) + [0] * (5 - len(shape))
    return ctypes.byref(_Shape(*f[:5]))


def _plan_dict(p) -> dict:
    d = {f: getattr(p, f) for f, _ in _Plan._fields_}
    d["kernel_name"] = KERNEL_NAMES.get(d["kernel"], "?")
    return d


def ggrms_forward_ex(y: int, gate: int, norm_weight: int, out: int, rows: int, width: int,
                     group_size: int, y_row_stride: int, gate_row_stride: int,
                     out_row_stride: int, eps: float, dtype: int, flags: int, stream: int) -> int:
    """The C entry point with operator flags (FLAG_ROUND_INTERMEDIATE,
    FLAG_NORM_BEFORE_GATE, FLAG_WEIGHT_PER_GROUP); returns the status."""
    return _lib.ggrms_forward_ex(y, gate, norm_weight, out, rows, width, group_size,
                                 y_row_stride, gate_row_stride, out_row_stride, eps, dtype, flags,
                                 stream)


def ggrms_forward_tuned(y: int, gate: int, norm_weight: int, out: int, rows: int, width: int,
                        group_size: int, y_row_stride: int, gate_row_stride: int,
                        out_row_stride: int, eps: float, dtype: int, flags: int, stream: int,
                        shape=None) -> int:
    """ggrms_forward_ex with launch controls: flags may also hold the FLAG_CACHE_*,
    FLAG_ORDER_* and FLAG_WAVE_* bits, and shape = (lanes, vectors[, rows per
    workgroup[, vector bytes[, kernel]]]) forces the kernel shape; returns the
    status."""
    return _lib.ggrms_forward_tuned(y, gate, norm_weight, out, rows, width, group_size,
                                    y_row_stride, gate_row_stride, out_row_stride, eps, dtype,
                                    flags, _shape_arg(shape), stream)


def ggrms_plan_tuned(y: int, gate: int, norm_weight: int, out: int, rows: int, width: int,
                     group_size: int, y_row_stride: int, gate_row_stride: int,
                     out_row_stride: int, eps: float, dtype: int, flags: int, shape=None):
    """(status, plan dict or None) for ggrms_forward_tuned's arguments; no device call."""
    p = _Plan()
    st = _lib.ggrms_plan_tuned(y, gate, norm_weight, out, rows, width, group_size, y_row_stride,
                               gate_row_stride, out_row_stride, eps, dtype, flags,
                               _shape_arg(shape), ctypes.byref(p))
    return (st, _plan_dict(p)) if st == SUCCESS else (st, None)


def ggrms_plan_ex(y: int, gate: int, norm_weight: int, out: int, rows: int, width: int,
                  group_size: int, y_row_stride: int, gate_row_stride: int, out_row_stride: int,
                  eps: float, dtype: int, flags: int):
    """(status, plan dict or None) for ggrms_forward_ex's arguments; no device call."""
    p = _Plan()
    st = _lib.ggrms_plan_ex(y, gate, norm_weight, out, rows, width, group_size, y_row_stride,
                            gate_row_stride, out_row_stride, eps, dtype, flags, ctypes.byref(p))
    return (st, _plan_dict(p)) if st == SUCCESS else (st, None)


def ggrms_plan(y: int, gate: int, norm_weight: int, out: int, rows: int, width: int,
               group_size: int, y_row_stride: int, gate_row_stride: int, out_row_stride: int,
               eps: float, dtype: int, round_intermediate: int):
    """(status, plan dict or None) -- the kernel ggrms_forward would launch; no device call."""
    p = _Plan()
    st = _lib.ggrms_plan(y, gate, norm_weight, out, rows, width, group_size, y_row_stride,
                         gate_row_stride, out_row_stride, eps, dtype, round_intermediate,
                         ctypes.byref(p))
    return (st, _plan_dict(p)) if st == SUCCESS else (st, None)


def ggrms_status_string(status: int) -> str:
    return _lib.ggrms_status_string(status).decode()


def ggrms_abi_version() -> int:
    return _lib.ggrms_abi_version()


# ----------------------------------------------------------- torch level

def _torch_dtype_code(t) -> int:
    import torch

    codes = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32, float16 or bfloat16")
    return codes[t.dtype]


def _as_rows(t, name: str):
    """View t (..., width) as rows with one row stride; returns (rows, row_stride)."""
    if t.dim() < 1:
        raise ValueError(f"{name} needs at least one dimension")
    if t.stride(-1) != 1 and t.size(-1) > 1:
        raise ValueError(f"{name} must have unit stride in its last dimension")
    width = t.size(-1)
    rows = t.numel() // width if width else 0
    if t.dim() == 1:
        return rows, width
    # leading axes must fold into a single row stride
    lead = [(s, st) for s, st in zip(t.shape[:-1], t.stride()[:-1]) if s != 1]
    if not lead:
        return rows, max(width, t.stride(-2))
    row_stride = lead[-1][1]
    expect = row_stride
    for s, st in reversed(lead):
        if st != expect:
            raise ValueError(f"{name}'s leading axes do not fold into one row stride")
        expect = st * s
    return rows, row_stride


def expand_head_scale(scale, heads: int):
    """A per-head scale of C elements shared by every head (any float dtype,
    shaped (C), (1, C) or (C, 1)) as the f32 per-column weight of heads*C
    columns.  The widening is exact; call once per weight, not per step."""
    s = scale.reshape(-1).float()
    return s.repeat(heads).contiguous()


def _weight_f32(weight, width: int, group_size: int):
    """The weight as the library takes it: a contiguous 1-D f32 tensor of
    width values (one per column) or group_size values (shared by every
    group).  Accepted spellings, after the Inputs table of the page
    "com.microsoft.GatedRMSNorm" (scale shaped (C), (1, C) or (C, 1)): 1-D,
    or 2-D with one axis of length 1; f32 as is, fp16/bf16 widened exactly
    (a copy per call: callers that repeat a call should widen once)."""
    import torch

    shape = tuple(weight.shape)
    if not (len(shape) == 1 or (len(shape) == 2 and 1 in shape)):
        raise ValueError(f"weight must be shaped (n), (1, n) or (n, 1), not {shape}")
    if weight.numel() not in (width, group_size):
        raise ValueError(f"weight has {weight.numel()} values; needs width ({width}) or "
                         f"group_size ({group_size})")
    if weight.dtype not in (torch.float32, torch.float16, torch.bfloat16):
        raise TypeError(f"unsupported weight dtype {weight.dtype}; use float32, float16 or "
                        "bfloat16")
    w = weight.reshape(-1)
    if w.dtype != torch.float32:
        w = w.float()  # every fp16 / bf16 value is an f32 value: exact
    return w if w.is_contiguous() else w.contiguous()


_CACHE_FLAGS = {None: 0, "stream": FLAG_CACHE_STREAM, "keep": FLAG_CACHE_KEEP}


def _flags(weight, width, group_size, round_intermediate, norm_before_gate, cache=None) -> int:
    if round_intermediate is None:
        round_intermediate = not norm_before_gate
    if cache not in _CACHE_FLAGS:
        raise ValueError(f"cache must be None, 'stream' or 'keep', not {cache!r}")
    per_group = weight.numel() == group_size and group_size != width
    return ((FLAG_ROUND_INTERMEDIATE if round_intermediate else 0) |
            (FLAG_NORM_BEFORE_GATE if norm_before_gate else 0) |
            (FLAG_WEIGHT_PER_GROUP if per_group else 0) | _CACHE_FLAGS[cache])


def forward(y, gate, weight, group_size: int, eps: float = 1e-5,
            round_intermediate=None, out=None, stream=None,
            norm_before_gate: bool = False, cache=None):
    """out = fused gated group-RMSNorm of (y, gate) with ``weight`` over groups
    of ``group_size`` columns of the last axis.

    y and gate: same shape (..., width), same dtype (f32/f16/bf16), on the
    GPU, unit stride in the last axis (they may be strided column slices of
    one fused buffer).  weight: width values (one per column) or group_size
    values (shared by every group), shaped (n), (1, n) or (n, 1), in f32 or
    (widened exactly to f32 here) fp16/bf16.  out (optional) must match y's
    shape and dtype; it is allocated like y when omitted.
    round_intermediate (default: on for gate first) casts gated*nf to the
    dtype before the weight multiply.  norm_before_gate selects
    out = ((y * nf) * w) * silu(gate) with nf from y alone, every
    intermediate f32 (round_intermediate=True is then refused).
    cache: None (the library streams jobs of at least STREAM_MIN_BYTES and
    keeps smaller ones cached), "stream" or "keep"; results are identical.
    Enqueued on ``stream`` (default: torch's current stream); no
    synchronisation.
    """
    import torch

    if y.shape != gate.shape:
        raise ValueError(f"y {tuple(y.shape)} and gate {tuple(gate.shape)} differ in shape")
    if y.dtype != gate.dtype:
        raise TypeError("y and gate must share a dtype")
    code = _torch_dtype_code(y)
    width = y.size(-1)
    if out is None:
        out = torch.empty(y.shape, dtype=y.dtype, device=y.device)
    elif out.shape != y.shape or out.dtype != y.dtype:
        raise ValueError("out must have y's shape and dtype")
    if not (y.is_cuda and gate.is_cuda and weight.is_cuda and out.is_cuda):
        raise ValueError("all tensors must be on the GPU")
    weight = _weight_f32(weight, width, group_size)
    rows, sy = _as_rows(y, "y")
    _, sg = _as_rows(gate, "gate")
    _, so = _as_rows(out, "out")
    if stream is None:
        stream = torch.cuda.current_stream(y.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    flags = _flags(weight, width, group_size, round_intermediate, norm_before_gate, cache)
    call = ggrms_forward_tuned if cache is not None else ggrms_forward_ex
    with torch.cuda.device(y.device):
        st = call(y.data_ptr(), gate.data_ptr(), weight.data_ptr(), out.data_ptr(), rows, width,
                  group_size, sy, sg, so, float(eps), code, flags, stream)
    if st != SUCCESS:
        raise GgrmsError(st)
    return out


def plan(y, gate, weight, group_size: int, eps: float = 1e-5, round_intermediate=None,
         out=None, norm_before_gate: bool = False, cache=None) -> dict:
    """The kernel forward() would launch for these tensors (no device call)."""
    code = _torch_dtype_code(y)
    width = y.size(-1)
    rows, sy = _as_rows(y, "y")
    _, sg = _as_rows(gate, "gate")
    o = out if out is not None else y.new_empty(y.shape)
    _, so = _as_rows(o, "out")
    weight = _weight_f32(weight, width, group_size)
    st, p = ggrms_plan_tuned(y.data_ptr(), gate.data_ptr(), weight.data_ptr(), o.data_ptr(), rows,
                             width, group_size, sy, sg, so, float(eps), code,
                             _flags(weight, width, group_size, round_intermediate,
                                    norm_before_gate, cache))
    if st != SUCCESS:
        raise GgrmsError(st, "ggrms_plan")
    return p
