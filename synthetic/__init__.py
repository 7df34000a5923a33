"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the method: it only draws numbers.  Each
value is a pure function of (seed, tensor id, flat element index) -- a
counter-based generator -- so any subset of rows can be regenerated without
generating the rest.

Generator (``synth.c``, built with gcc): SplitMix64 (Steele, Lea and Flood,
"Fast splittable pseudorandom number generators", OOPSLA 2014) used as a hash
of the counter; normals by the Box-Muller transform (cosine branch) in
double, rounded once to float32; the float32 draw goes to the storage dtype
by torch's CPU cast.  Neither the oracle nor the HIP library is involved.
"""
from __future__ import annotations

import concurrent.futures as _cf
import ctypes
import dataclasses
import os
import subprocess

import numpy as np

F32, F16, BF16 = 0, 1, 2
DTYPE_NAMES = {F32: "f32", F16: "f16", BF16: "bf16"}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")


def build(force: bool = True) -> str:
    """Compile the draw routines with gcc into ``synthetic/libsynth.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"],
                       check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _L():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        u64, i64, vp, d = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
        L.synth_normal_f32.argtypes = [u64, u64, u64, i64, d, vp]
        L.synth_uniform_f32.argtypes = [u64, u64, u64, i64, d, d, vp]
        L.synth_rows_f32.argtypes = [u64, u64, vp, i64, i64, ctypes.c_int, d, d, vp]
        _lib = L
    return _lib


def _draw_f32(seed: int, tensor_id: int, first: int, n: int, dist: tuple) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    if dist[0] == "normal":
        _L().synth_normal_f32(seed, tensor_id, first, n, float(dist[1]), out.ctypes.data)
    else:
        _L().synth_uniform_f32(seed, tensor_id, first, n, float(dist[1]), float(dist[2]),
                               out.ctypes.data)
    return out


def to_storage(x32: np.ndarray, dtype: int) -> np.ndarray:
    """float32 draws -> storage array (float32, or uint16 bit patterns for
    fp16/bf16) by torch's CPU cast (round to nearest even)."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == F32:
        return x32
    import torch  # CPU cast only

    tdt = torch.float16 if dtype == F16 else torch.bfloat16
    return torch.from_numpy(x32).to(tdt).view(torch.int16).numpy().view(np.uint16)


def storage_dtype(dtype: int):
    return np.float32 if dtype == F32 else np.uint16


def tensor(seed: int, tensor_id: int, n: int, dtype: int, dist: tuple,
           chunk: int = 1 << 22) -> np.ndarray:
    """Flat storage array of draws 0..n-1; dist = ("normal", sigma) or ("uniform", lo, hi)."""
    out = np.empty(n, dtype=storage_dtype(dtype))

    def work(s):
        e = min(s + chunk, n)
        out[s:e] = to_storage(_draw_f32(seed, tensor_id, s, e - s, dist), dtype)

    starts = list(range(0, n, chunk))
    if len(starts) <= 1:
        for s in starts:
            work(s)
        return out
    with _cf.ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(work, starts))
    return out


def tensor_rows(seed: int, tensor_id: int, row_len: int, rows, dtype: int,
                dist: tuple) -> np.ndarray:
    """Rows `rows` of a [*, row_len] tensor drawn by `tensor`, as [len(rows), row_len]."""
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty(len(rows) * row_len, dtype=np.float32)
    kind = 0 if dist[0] == "normal" else 1
    p1 = float(dist[2]) if kind else 0.0
    _L().synth_rows_f32(seed, tensor_id, rows.ctypes.data, len(rows), row_len, kind,
                        float(dist[1]), p1, out.ctypes.data)
    return to_storage(out, dtype).reshape(len(rows), row_len)


# ------------------------------------------------------------------ workloads

TID_Y, TID_GATE, TID_W = 1, 2, 3
BASE_SEED = 20261202


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, dtypes, distributions and layout."""

    name: str
    index: int
    rows: int
    width: int
    group_size: int
    dtype: int
    eps: float
    round_intermediate: int
    act_dist: tuple
    weight_dist: tuple = ("uniform", 0.5, 1.5)
    # Fused in-proj layout: y and gate are column slices of one [rows, fused_width]
    # buffer at columns y_col and gate_col; 0 means separate contiguous tensors.
    fused_width: int = 0
    y_col: int = 0
    gate_col: int = 0
    # Per-head scale of scale_len elements shared by every head, stored in
    # scale_dtype and expanded to the f32 per-column weight (0 = per-column weight).
    scale_len: int = 0
    scale_dtype: int = F32

    @property
    def seed(self) -> int:
        return BASE_SEED + self.index

    @property
    def groups(self) -> int:
        return self.width // self.group_size

    @property
    def esize(self) -> int:
        return 4 if self.dtype == F32 else 2

    def algorithmic_bytes(self, per_group_weight: bool = False) -> int:
        """y, gate and out each touched once, plus the f32 weight once (width
        values, or group_size values when one weight is shared by every group)."""
        wlen = self.group_size if per_group_weight else self.width
        return 3 * self.rows * self.width * self.esize + 4 * wlen


WORKLOADS = {
    "tiny_4x256_f32_g64": Workload(
        "tiny_4x256_f32_g64", 0, 4, 256, 64, F32, 1e-5, 0, ("normal", 1.0)),
    "mamba2_decode_1x7680_bf16_g960": Workload(
        "mamba2_decode_1x7680_bf16_g960", 1, 1, 7680, 960, BF16, 1e-5, 1, ("normal", 1.0)),
    "strided_256x4800_f16_g100": Workload(
        "strided_256x4800_f16_g100", 2, 256, 4800, 100, F16, 1e-5, 1, ("normal", 1.0),
        fused_width=9856, y_col=0, gate_col=4800),
    "mamba2_prefill_8192x7680_bf16_g960": Workload(
        "mamba2_prefill_8192x7680_bf16_g960", 3, 8192, 7680, 960, BF16, 1e-5, 1,
        ("normal", 2.0)),
    "gdn_head_16384x8192_f16_g128": Workload(
        "gdn_head_16384x8192_f16_g128", 4, 16384, 8192, 128, F16, 1e-6, 0, ("normal", 1.0),
        scale_len=128, scale_dtype=F16),
}

# Decode replays 21 layers back to back, each with its own inputs.
DECODE_LAYERS = 21


def fused_sentinel_value(dtype: int):
    """Bit pattern written into the never-read columns of a fused buffer (a quiet NaN)."""
    return {F32: np.float32(np.nan), F16: np.uint16(0x7E00), BF16: np.uint16(0x7FC0)}[dtype]


def make_weight(w: Workload, layer: int = 0) -> np.ndarray:
    """The f32 per-column norm weight, [width].  For a per-head scale it is the
    scale drawn in its own dtype, widened exactly and tiled over the heads."""
    seed = w.seed + 1000 * layer
    if w.scale_len:
        s = tensor(seed, TID_W, w.scale_len, w.scale_dtype, w.weight_dist)
        if w.scale_dtype != F32:
            import torch

            tdt = torch.float16 if w.scale_dtype == F16 else torch.bfloat16
            s = torch.from_numpy(s.view(np.int16)).view(tdt).float().numpy()
        return np.tile(s.astype(np.float32), w.width // w.scale_len)
    return tensor(seed, TID_W, w.width, F32, w.weight_dist)


def make_inputs(w: Workload, layer: int = 0):
    """Host inputs for workload w.

    Returns (y_buf, gate_buf, weight, layout) where layout is a dict with
    y_offset, gate_offset, y_row_stride, gate_row_stride (elements).  For a
    fused layout y_buf is gate_buf (one [rows, fused_width] buffer with NaN in
    the columns neither slice covers)."""
    seed = w.seed + 1000 * layer
    n = w.rows * w.width
    weight = make_weight(w, layer)
    if w.fused_width:
        fw = w.fused_width
        yv = tensor(seed, TID_Y, n, w.dtype, w.act_dist).reshape(w.rows, w.width)
        gv = tensor(seed, TID_GATE, n, w.dtype, w.act_dist).reshape(w.rows, w.width)
        buf = np.empty((w.rows, fw), dtype=storage_dtype(w.dtype))
        buf[:] = fused_sentinel_value(w.dtype)
        buf[:, w.y_col:w.y_col + w.width] = yv
        buf[:, w.gate_col:w.gate_col + w.width] = gv
        flat = buf.reshape(-1)
        layout = dict(y_offset=w.y_col, gate_offset=w.gate_col, y_row_stride=fw,
                      gate_row_stride=fw)
        return flat, flat, weight, layout
    y = tensor(seed, TID_Y, n, w.dtype, w.act_dist)
    g = tensor(seed, TID_GATE, n, w.dtype, w.act_dist)
    layout = dict(y_offset=0, gate_offset=0, y_row_stride=w.width, gate_row_stride=w.width)
    return y, g, weight, layout


def make_rows(w: Workload, rows: np.ndarray, layer: int = 0):
    """Rows `rows` of y and gate as contiguous [len(rows), width] arrays
    (identical to the same rows of make_inputs)."""
    seed = w.seed + 1000 * layer
    y = tensor_rows(seed, TID_Y, w.width, rows, w.dtype, w.act_dist)
    g = tensor_rows(seed, TID_GATE, w.width, rows, w.dtype, w.act_dist)
    return y, g
