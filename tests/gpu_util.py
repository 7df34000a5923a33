"""Helpers shared by the GPU parity tests: device buffers from the seeded
host arrays, the parity bar, and calls through the C ABI."""
import numpy as np
import torch

import synthetic as S

F32, F16, BF16 = 0, 1, 2
TDT = {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16}
DT_IDS = {F32: "f32", F16: "f16", BF16: "bf16"}
FLAG_RI, FLAG_NBG, FLAG_PER_GROUP, FLAG_STREAM, FLAG_KEEP = 1, 2, 4, 8, 16


def say(msg):
    print(msg, flush=True)


# ------------------------------------------------------------ helpers

def dev_buf(host: np.ndarray, dtype: int) -> torch.Tensor:
    """Flat device tensor holding the storage array's bits."""
    t = torch.from_numpy(np.ascontiguousarray(host).view(np.int16) if dtype != F32 else
                         np.ascontiguousarray(host))
    t = t.view(TDT[dtype]) if dtype != F32 else t
    return t.reshape(-1).to("cuda")


def host_bits(t: torch.Tensor, dtype: int) -> np.ndarray:
    c = t.detach().cpu().reshape(-1)
    if dtype == F32:
        return c.numpy()
    return c.view(torch.int16).numpy().view(np.uint16)


def ulp_key(b):
    b = b.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)


def nan16(b, dtype):
    b = b.astype(np.int64)
    if dtype == F16:
        return ((b & 0x7C00) == 0x7C00) & ((b & 0x3FF) != 0)
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)


def assert_parity(got: np.ndarray, ref: np.ndarray, dtype: int, what: str = "") -> dict:
    """The parity bar; returns statistics."""
    assert got.shape == ref.shape
    if dtype == F32:
        g64 = got.astype(np.float64)
        r64 = ref.astype(np.float64)
        gn, rn = np.isnan(g64), np.isnan(r64)
        assert np.array_equal(gn, rn), f"{what}: NaN positions differ ({int((gn != rn).sum())})"
        ok = ~rn
        # equal values (infinities included) differ by 0, not by inf - inf
        with np.errstate(invalid="ignore"):
            err = np.where(g64[ok] == r64[ok], 0.0, np.abs(g64[ok] - r64[ok]))
        lim = 1e-5 * np.abs(r64[ok])
        # a zero reference needs a zero (or an underflowed f32 subnormal) result
        lim = np.where(r64[ok] == 0, 2.0 ** -126, lim)
        bad = err > lim
        assert not bad.any(), (f"{what}: {int(bad.sum())} f32 outputs off by more than 1e-5 "
                               f"relative; worst {float((err / np.maximum(np.abs(r64[ok]), 1e-38)).max()):.3e}")
        rel = err / np.maximum(np.abs(r64[ok]), 1e-38)
        return {"max_rel": float(rel.max()) if rel.size else 0.0,
                "exact": float((got[ok].view(np.uint32) == ref[ok].view(np.uint32)).mean()) if ok.any() else 1.0}
    gn, rn = nan16(got, dtype), nan16(ref, dtype)
    assert np.array_equal(gn, rn), f"{what}: NaN positions differ ({int((gn != rn).sum())})"
    ok = ~rn
    d = np.abs(ulp_key(got[ok]) - ulp_key(ref[ok]))
    if d.size:
        i = int(np.argmax(d))
        assert d.max() <= 2, (f"{what}: {int((d > 2).sum())} outputs beyond 2 ulp; worst {int(d.max())} "
                              f"(got {got[ok][i]:#06x}, oracle {ref[ok][i]:#06x})")
    return {"max_ulp": int(d.max()) if d.size else 0, "exact": float((d == 0).mean()) if d.size else 1.0}


def run_gpu(g, y, gate, w, out, rows, width, G, sy, sg, so, eps, dtype, ri, shape=None,
            stream=None, flags=None):
    """y/gate/out: device tensors (already offset views allowed); returns the
    status.  No flags and no shape: ggrms_forward.  Operator flags only
    (FLAG_RI, FLAG_NBG, FLAG_PER_GROUP): ggrms_forward_ex.  Launch controls
    among the flags, or a forced shape (lanes, vectors[, rows per
    workgroup[, vector bytes]]): ggrms_forward_tuned, with ri as FLAG_RI when
    flags is None."""
    s = (stream or torch.cuda.current_stream()).cuda_stream
    if flags is None and shape is None:
        return g.ggrms_forward(y.data_ptr(), gate.data_ptr(), w.data_ptr(), out.data_ptr(), rows,
                               width, G, sy, sg, so, eps, dtype, ri, s)
    if flags is None:
        flags = FLAG_RI if ri else 0
    if shape is None and not flags & ~(FLAG_RI | FLAG_NBG | FLAG_PER_GROUP):
        return g.ggrms_forward_ex(y.data_ptr(), gate.data_ptr(), w.data_ptr(), out.data_ptr(),
                                  rows, width, G, sy, sg, so, eps, dtype, flags, s)
    return g.ggrms_forward_tuned(y.data_ptr(), gate.data_ptr(), w.data_ptr(), out.data_ptr(),
                                 rows, width, G, sy, sg, so, eps, dtype, flags, s, shape)


def random_case(rows, width, dtype, seed, dist=("normal", 1.0), gate_dist=None):
    n = rows * width
    y = S.tensor(seed, S.TID_Y, n, dtype, dist)
    gt = S.tensor(seed, S.TID_GATE, n, dtype, gate_dist or dist)
    w = S.tensor(seed, S.TID_W, width, F32, ("uniform", 0.5, 1.5))
    return y, gt, w


def check_contiguous(g, orc, rows, width, G, dtype, ri, seed, eps=1e-5, shape=None,
                     dist=("normal", 1.0), gate_dist=None, tag="", flags=None):
    """One contiguous [rows, width] case through the GPU and the oracle.
    With flags (FLAG_* mask) the case goes through ggrms_forward_tuned and, for
    FLAG_PER_GROUP, the weight is the first G values of the drawn one."""
    say(f"case {tag} rows={rows} width={width} G={G} dtype={DT_IDS[dtype]} ri={ri} "
        f"flags={flags} shape={shape}")
    y, gt, w = random_case(rows, width, dtype, seed, dist, gate_dist)
    per_group = bool(flags and flags & FLAG_PER_GROUP)
    if per_group:
        w = np.ascontiguousarray(w[:G])
    yd, gd, wd = dev_buf(y, dtype), dev_buf(gt, dtype), torch.from_numpy(w).cuda()
    od = torch.empty_like(yd)
    st = run_gpu(g, yd, gd, wd, od, rows, width, G, width, width, width, eps, dtype, ri, shape,
                 flags=flags)
    assert st == g.SUCCESS, g.ggrms_status_string(st)
    torch.cuda.synchronize()
    got = host_bits(od, dtype)
    if flags is not None:
        ri = flags & FLAG_RI
    ref = orc.forward(y, gt, w, rows=rows, width=width, group_size=G, y_row_stride=width,
                      gate_row_stride=width, out_row_stride=width, eps=eps, dtype=dtype,
                      round_intermediate=ri, norm_before_gate=bool(flags and flags & FLAG_NBG),
                      weight_per_group=per_group)
    return assert_parity(got, ref, dtype, tag)
