"""CPU oracle for the fused gated group-RMSNorm -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does.

The arithmetic lives in ``ggrms_oracle.c`` (plain C, single-threaded, f32 as
the "gated_group_rmsnorm" page's math block prescribes, explicit
round-to-nearest-even casts).  This module only builds it with gcc and
marshals numpy arrays into it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ggrms_oracle.c")
_LIB = os.path.join(_HERE, "libggrms_oracle.so")

F32, F16, BF16 = 0, 1, 2
ROUND_INTERMEDIATE, NORM_BEFORE_GATE, WEIGHT_PER_GROUP = 1, 2, 4
_NP_STORAGE = {F32: np.float32, F16: np.uint16, BF16: np.uint16}

# Strict IEEE f32: no contraction into fused multiply-add, no fast-math,
# SSE arithmetic (the x86-64 default), no flush-to-zero.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-fno-unsafe-math-optimizations", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/libggrms_oracle.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        L.ggrms_oracle_forward.restype = ctypes.c_int
        L.ggrms_oracle_forward.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                           ctypes.c_float, ctypes.c_int, ctypes.c_int, vp]
        L.ggrms_oracle_forward_ex.restype = ctypes.c_int
        L.ggrms_oracle_forward_ex.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                              ctypes.c_float, ctypes.c_int, ctypes.c_int, vp]
        L.ggrms_oracle_silu.restype = ctypes.c_float
        L.ggrms_oracle_silu.argtypes = [ctypes.c_float]
        L.ggrms_oracle_round_array.argtypes = [vp, vp, i64, ctypes.c_int]
        L.ggrms_oracle_round_bits_range.argtypes = [ctypes.c_uint32, i64, vp, ctypes.c_int]
        L.ggrms_oracle_widen_array.argtypes = [vp, vp, i64, ctypes.c_int]
        L.ggrms_oracle_silu_array.argtypes = [vp, vp, i64]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def forward(y: np.ndarray, gate: np.ndarray, weight: np.ndarray, *, rows: int, width: int,
            group_size: int, y_row_stride: int, gate_row_stride: int, out_row_stride: int,
            eps: float, dtype: int, round_intermediate: int = 0,
            out: np.ndarray | None = None, y_offset: int = 0, gate_offset: int = 0,
            out_offset: int = 0, norm_before_gate: bool = False,
            weight_per_group: bool = False) -> np.ndarray:
    """Run the oracle on flat host buffers.

    ``y``/``gate``/``out`` are 1-D numpy buffers of the storage type
    (float32, or uint16 bit patterns for fp16/bf16); the offsets and row
    strides are in elements, so strided column slices of one fused buffer
    are passed as the same array with different offsets.  ``weight`` has
    ``width`` values, or ``group_size`` with ``weight_per_group``.
    """
    st = _NP_STORAGE[dtype]
    for name, a in (("y", y), ("gate", gate)):
        if a.dtype != st or a.ndim != 1 or not a.flags.c_contiguous:
            raise TypeError(f"{name} must be a contiguous 1-D {np.dtype(st).name} array")
    weight = np.ascontiguousarray(weight, dtype=np.float32)
    if weight.size < (group_size if weight_per_group else width):
        raise ValueError("weight too short")
    if rows > 0:
        need = lambda off, s: off + (rows - 1) * s + width
        if need(y_offset, y_row_stride) > y.size or need(gate_offset, gate_row_stride) > gate.size:
            raise ValueError("input buffer too small for rows/strides")
    if out is None:
        out = np.zeros(out_offset + max(rows - 1, 0) * out_row_stride + width if rows else 0,
                       dtype=st)
    elif rows > 0 and out_offset + (rows - 1) * out_row_stride + width > out.size:
        raise ValueError("out buffer too small")
    scratch = np.empty(max(group_size, 1), dtype=np.float32)
    es = np.dtype(st).itemsize
    flags = ((ROUND_INTERMEDIATE if round_intermediate else 0) |
             (NORM_BEFORE_GATE if norm_before_gate else 0) |
             (WEIGHT_PER_GROUP if weight_per_group else 0))
    if round_intermediate not in (0, 1, True, False):
        raise ValueError("round_intermediate must be 0 or 1")
    rc = lib().ggrms_oracle_forward_ex(
        _ptr(y) + y_offset * es, _ptr(gate) + gate_offset * es, _ptr(weight),
        _ptr(out) + out_offset * es, rows, width, group_size, y_row_stride,
        gate_row_stride, out_row_stride, ctypes.c_float(eps), dtype, flags, _ptr(scratch))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out


def forward_2d(y: np.ndarray, gate: np.ndarray, weight: np.ndarray, group_size: int,
               eps: float, dtype: int, round_intermediate: int, norm_before_gate: bool = False,
               weight_per_group: bool = False) -> np.ndarray:
    """Contiguous ``[rows, width]`` convenience wrapper; returns ``[rows, width]``."""
    rows, width = y.shape
    out = forward(np.ascontiguousarray(y).reshape(-1), np.ascontiguousarray(gate).reshape(-1),
                  weight, rows=rows, width=width, group_size=group_size, y_row_stride=width,
                  gate_row_stride=width, out_row_stride=width, eps=eps, dtype=dtype,
                  round_intermediate=round_intermediate, norm_before_gate=norm_before_gate,
                  weight_per_group=weight_per_group)
    return out.reshape(rows, width)


def round_to(x: np.ndarray, dtype: int) -> np.ndarray:
    """f32 array -> uint16 bit patterns (fp16 or bf16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().ggrms_oracle_round_array(_ptr(x), _ptr(out), x.size, dtype)
    return out


def round_bits_range(first: int, n: int, dtype: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    lib().ggrms_oracle_round_bits_range(first, n, _ptr(out), dtype)
    return out


def widen(h: np.ndarray, dtype: int) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    lib().ggrms_oracle_widen_array(_ptr(h), _ptr(out), h.size, dtype)
    return out


def silu(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.float32)
    lib().ggrms_oracle_silu_array(_ptr(x), _ptr(out), x.size)
    return out
