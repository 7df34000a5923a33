"""Fused gated group-RMSNorm for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libggrms.so`` (C ABI in ``include/ggrms.h``).
Every step of the computation runs in the library's HIP kernels; this
module only marshals arguments.  PyTorch supplies device memory and the
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
    "ERROR_INVALID_VALUE", "ERROR_NOT_SUPPORTED", "ERROR_LAUNCH", "KERNEL_NAMES", "GgrmsError", "ggrms_forward", "ggrms_forward_ex",
    "ggrms_forward_with_shape", "ggrms_plan", "ggrms_plan_ex",
    "ggrms_status_string", "ggrms_abi_version", "forward", "plan", "expand_head_scale",
    "library_path",
]

F32, F16, BF16 = 0, 1, 2
FLAG_ROUND_INTERMEDIATE, FLAG_NORM_BEFORE_GATE, FLAG_WEIGHT_PER_GROUP = 1, 2, 4
FLAG_CACHE_STREAM, FLAG_CACHE_KEEP = 8, 16
# launch controls (tile order, WAVE workgroup size); results are identical whatever they select
FLAG_ORDER_ROWS, FLAG_ORDER_BANDED, FLAG_WAVE_ONE, FLAG_WAVE_FOUR = 32, 64, 128, 256
STREAM_MIN_BYTES = 4 << 20  # default policy: jobs of at least this many y+gate+out bytes stream
SUCCESS, ERROR_INVALID_VALUE, ERROR_NOT_SUPPORTED, ERROR_LAUNCH = 0, 1, 2, 3
KERNEL_NAMES = {0: "none", 1: "wave", 2: "block", 3: "wide"}
ABI_VERSION = 4

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
                ("rows_per_workgroup", ctypes.c_int32)]


class _Plan(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("vector_bytes", ctypes.c_int32),
                ("lanes_per_group", ctypes.c_int32), ("vectors_per_lane", ctypes.c_int32),
                ("block_threads", ctypes.c_int32), ("launches", ctypes.c_int32),
                ("rows_per_workgroup", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
                ("workgroups", ctypes.c_int64), ("streaming", ctypes.c_int32),
                ("piece_bytes", ctypes.c_int32), ("tile_order", ctypes.c_int32)]


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
    L.ggrms_forward_with_shape.argtypes = fwd + [i32, i32, i32, vp]
    L.ggrms_forward_with_shape.restype = i32
    L.ggrms_plan.argtypes = fwd + [ctypes.POINTER(_Plan)]
    L.ggrms_plan.restype = i32
    fwd_ex = fwd[:-1] + [ctypes.c_uint32, ctypes.POINTER(_Shape)]
    L.ggrms_forward_ex.argtypes = fwd_ex + [vp]
    L.ggrms_forward_ex.restype = i32
    L.ggrms_plan_ex.argtypes = fwd_ex + [ctypes.POINTER(_Plan)]
    L.ggrms_plan_ex.restype = i32
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


def ggrms_forward_with_shape(y: int, gate: int, norm_weight: int, out: int, rows: int,
                             width: int, group_size: int, y_row_stride: int,
                             gate_row_stride: int, out_row_stride: int, eps: float, dtype: int,
                             round_intermediate: int, lanes_per_group: int,
                             vectors_per_lane: int, stream: int,
                             rows_per_workgroup: int = 0) -> int:
    """ggrms_forward with a caller-chosen kernel shape; returns the status."""
    return _lib.ggrms_forward_with_shape(y, gate, norm_weight, out, rows, width, group_size,
                                         y_row_stride, gate_row_stride, out_row_stride, eps,
                                         dtype, round_intermediate, lanes_per_group,
                                         vectors_per_lane, rows_per_workgroup, stream)


def _shape_arg(shape):
    if shape is None:
        return None
    lanes, vpt = shape[0], shape[1]
    upb = shape[2] if len(shape) > 2 else 0
    return ctypes.byref(_Shape(lanes, vpt, upb))


def ggrms_forward_ex(y: int, gate: int, norm_weight: int, out: int, rows: int, width: int,
                     group_size: int, y_row_stride: int, gate_row_stride: int,
                     out_row_stride: int, eps: float, dtype: int, flags: int, stream: int,
                     shape=None) -> int:
    """The C entry point with operator flags and an optional (lanes, vectors[, rows
    per workgroup]) shape; returns the status."""
    return _lib.ggrms_forward_ex(y, gate, norm_weight, out, rows, width, group_size,
                                 y_row_stride, gate_row_stride, out_row_stride, eps, dtype, flags,
                                 _shape_arg(shape), stream)


def ggrms_plan_ex(y: int, gate: int, norm_weight: int, out: int, rows: int, width: int,
                  group_size: int, y_row_stride: int, gate_row_stride: int, out_row_stride: int,
                  eps: float, dtype: int, flags: int, shape=None):
    """(status, plan dict or None) for ggrms_forward_ex's arguments; no device call."""
    p = _Plan()
    st = _lib.ggrms_plan_ex(y, gate, norm_weight, out, rows, width, group_size, y_row_stride,
                            gate_row_stride, out_row_stride, eps, dtype, flags,
                            _shape_arg(shape), ctypes.byref(p))
    if st != SUCCESS:
        return st, None
    d = {f: getattr(p, f) for f, _ in _Plan._fields_}
    d["kernel_name"] = KERNEL_NAMES.get(d["kernel"], "?")
    return st, d


def ggrms_plan(y: int, gate: int, norm_weight: int, out: int, rows: int, width: int,
               group_size: int, y_row_stride: int, gate_row_stride: int, out_row_stride: int,
               eps: float, dtype: int, round_intermediate: int):
    """(status, plan dict or None) -- the kernel ggrms_forward would launch; no device call."""
    p = _Plan()
    st = _lib.ggrms_plan(y, gate, norm_weight, out, rows, width, group_size, y_row_stride,
                         gate_row_stride, out_row_stride, eps, dtype, round_intermediate,
                         ctypes.byref(p))
    if st != SUCCESS:
        return st, None
    d = {f: getattr(p, f) for f, _ in _Plan._fields_}
    d["kernel_name"] = KERNEL_NAMES.get(d["kernel"], "?")
    return st, d


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
    """out = fused gated group-RMSNorm of (y, gate) with the f32 ``weight``
    over groups of ``group_size`` columns of the last axis.

    y and gate: same shape (..., width), same dtype (f32/f16/bf16), on the
    GPU, unit stride in the last axis (they may be strided column slices of
    one fused buffer).  weight: f32 with width values (one per column) or
    group_size values (shared by every group).  out (optional) must match
    y's shape and dtype; it is allocated like y when omitted.
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
    if weight.dtype != torch.float32 or weight.dim() != 1 or \
            weight.numel() not in (width, group_size):
        raise TypeError("weight must be a 1-D float32 tensor with width or group_size elements "
                        "(expand_head_scale builds a per-column one from a per-head scale)")
    if not weight.is_contiguous():
        raise ValueError("weight must be contiguous")
    if out is None:
        out = torch.empty(y.shape, dtype=y.dtype, device=y.device)
    elif out.shape != y.shape or out.dtype != y.dtype:
        raise ValueError("out must have y's shape and dtype")
    if not (y.is_cuda and gate.is_cuda and weight.is_cuda and out.is_cuda):
        raise ValueError("all tensors must be on the GPU")
    rows, sy = _as_rows(y, "y")
    _, sg = _as_rows(gate, "gate")
    _, so = _as_rows(out, "out")
    if stream is None:
        stream = torch.cuda.current_stream(y.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    flags = _flags(weight, width, group_size, round_intermediate, norm_before_gate, cache)
    with torch.cuda.device(y.device):
        st = ggrms_forward_ex(y.data_ptr(), gate.data_ptr(), weight.data_ptr(), out.data_ptr(),
                              rows, width, group_size, sy, sg, so, float(eps), code, flags,
                              stream)
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
    st, p = ggrms_plan_ex(y.data_ptr(), gate.data_ptr(), weight.data_ptr(), o.data_ptr(), rows,
                          width, group_size, sy, sg, so, float(eps), code,
                          _flags(weight, width, group_size, round_intermediate,
                                 norm_before_gate, cache))
    if st != SUCCESS:
        raise GgrmsError(st, "ggrms_plan")
    return p
