"""Independent references and comparison rules used by the tests.

Nothing here calls the oracle or the HIP library.  The references are:

* ``chain_fp64`` -- the unfused op chain that the "gated_group_rmsnorm" page's
  intro says the fused op replaces (widen, silu-gate, group RMSNorm, weight
  multiply and narrow), built from library routines (torch.nn.functional.silu
  and torch.nn.functional.rms_norm) evaluated in float64;
* ``exact_unit`` -- the page's math block evaluated with Python's decimal
  module at 60 significant digits (brute force for tiny inputs);
* casts between storage bit patterns and float64 through torch's CPU casts.

Comparison rule for 16-bit outputs: the oracle computes in f32, so its value
before each cast may differ from the exact one by a relative ``delta`` (an
error bound derived from the f32 arithmetic).  Where the exact value lies
more than ``delta`` away from every rounding boundary of the target format,
the cast result is fixed and the oracle must match it bit for bit; elsewhere
it may land on either neighbour (one unit in the last place per cast).
"""
from __future__ import annotations

import decimal

import numpy as np
import torch

F32, F16, BF16 = 0, 1, 2
U32 = 2.0 ** -24  # unit roundoff of binary32
_TDT = {F16: torch.float16, BF16: torch.bfloat16, F32: torch.float32}


def widen64(a: np.ndarray, dtype: int) -> np.ndarray:
    """Storage (float32 or uint16 bits) -> float64, exactly (torch CPU casts)."""
    if dtype == F32:
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(_TDT[dtype])
    return t.double().numpy()


def round64(x: np.ndarray, dtype: int) -> np.ndarray:
    """float64 -> storage of dtype, round to nearest even (torch CPU cast)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    if dtype == F32:
        return t.float().numpy()
    return t.to(_TDT[dtype]).view(torch.int16).numpy().view(np.uint16)


def _neighbours(bits: np.ndarray, dtype: int):
    """Values just below and just above each representable value (by magnitude order)."""
    b = bits.astype(np.int64)
    sign = b & 0x8000
    mag = b & 0x7FFF
    up = np.where(mag < 0x7FFF, mag + 1, mag) | sign
    dn = np.where(mag > 0, mag - 1, mag) | sign
    return widen64(dn.astype(np.uint16), dtype), widen64(up.astype(np.uint16), dtype)


def near_tie(x: np.ndarray, dtype: int, delta) -> np.ndarray:
    """True where x is within relative delta of a rounding boundary of dtype."""
    x = np.asarray(x, dtype=np.float64)
    r_bits = round64(x, dtype)
    r = widen64(r_bits, dtype)
    dn, up = _neighbours(r_bits, dtype)
    with np.errstate(invalid="ignore", over="ignore"):
        m1 = (r + dn) / 2.0
        m2 = (r + up) / 2.0
        band = np.abs(x) * delta
        near = (np.abs(x - m1) <= band) | (np.abs(x - m2) <= band)
    # zero-valued boundaries around 0 and the overflow threshold count as near too
    return near | ~np.isfinite(r)


def ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in units in the last place between 16-bit patterns (+0 == -0)."""
    def key(v):
        v = v.astype(np.int64)
        mag = v & 0x7FFF
        return np.where(v & 0x8000, -mag, mag)
    return np.abs(key(a) - key(b))


def is_nan16(bits: np.ndarray, dtype: int) -> np.ndarray:
    b = bits.astype(np.int64)
    if dtype == F16:
        return ((b & 0x7C00) == 0x7C00) & ((b & 0x03FF) != 0)
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)


def chain_fp64(yd: np.ndarray, gd: np.ndarray, group_size: int, eps: float) -> np.ndarray:
    """t = gated * rsqrt(mean(gated^2) + eps) per group, float64, via library routines.

    yd, gd: float64 [rows, width].  Returns float64 [rows, width]."""
    rows, width = yd.shape
    y = torch.from_numpy(yd)
    g = torch.from_numpy(gd)
    gated = y * torch.nn.functional.silu(g)
    t = torch.nn.functional.rms_norm(gated.reshape(rows, width // group_size, group_size),
                                     (group_size,), eps=eps)
    return t.reshape(rows, width).numpy()


def chain_nbg_fp64(yd: np.ndarray, gd: np.ndarray, w: np.ndarray, group_size: int,
                   eps: float) -> np.ndarray:
    """Norm before gate, float64, library routines: rms_norm(y) * w * silu(gate).

    w: float64 [width] (per column; tile a per-group weight first)."""
    rows, width = yd.shape
    t = torch.nn.functional.rms_norm(torch.from_numpy(yd).reshape(rows, width // group_size,
                                                                  group_size),
                                     (group_size,), eps=eps).reshape(rows, width)
    return (t * torch.from_numpy(w)[None, :] * torch.nn.functional.silu(torch.from_numpy(gd))).numpy()


def oracle_delta(group_size: int) -> float:
    """Relative error bound of the oracle's f32 value of gated*nf (and w*that)
    against the exact one: the f32 sum of G squares (<= (G+2)u), halved by the
    square root, plus a few roundings for silu, the division, eps, sqrt, the
    reciprocal and the products."""
    return (group_size / 2.0 + 16.0) * U32


def expected_16bit(t_exact: np.ndarray, w: np.ndarray, group_size: int, dtype: int, ri: int):
    """(expected output bits, mask where the oracle must match them exactly)."""
    delta = oracle_delta(group_size)
    if ri:
        t_bits = round64(t_exact, dtype)
        t_near = near_tie(t_exact, dtype, delta)
        p = w * widen64(t_bits, dtype)  # exact in float64
        p_near = near_tie(p, dtype, 4 * U32)  # the oracle's f32 product rounds once
    else:
        t_near = np.zeros(t_exact.shape, dtype=bool)
        p = w * t_exact
        p_near = near_tie(p, dtype, delta + 4 * U32)
    return round64(p, dtype), ~(t_near | p_near)


def check_16bit(out_bits: np.ndarray, t_exact: np.ndarray, w: np.ndarray, group_size: int,
                dtype: int, ri: int, min_exact_fraction: float = 0.6) -> dict:
    """Assert the tie-aware rule; returns a few statistics."""
    exp_bits, exact = expected_16bit(t_exact, w, group_size, dtype, ri)
    nan_o = is_nan16(out_bits, dtype)
    nan_e = is_nan16(exp_bits, dtype)
    assert np.array_equal(nan_o, nan_e), "NaN positions differ"
    ok = ~nan_e
    mism = (out_bits != exp_bits) & exact & ok
    # +0 and -0 are equal values
    mism &= ulp_distance(out_bits, exp_bits) != 0
    assert not mism.any(), (
        f"{int(mism.sum())} elements differ where the rounding is fixed; first at "
        f"{np.argwhere(mism)[0].tolist()}: got {out_bits[mism][0]:#06x} want {exp_bits[mism][0]:#06x}")
    d = ulp_distance(out_bits[ok], exp_bits[ok])
    assert d.size == 0 or d.max() <= 2, f"max ulp distance {d.max()}"
    frac = float(exact[ok].mean()) if ok.any() else 1.0
    assert frac >= min_exact_fraction, f"only {frac:.2%} of elements are tie-free"
    return {"exact_fraction": frac, "max_ulp": int(d.max()) if d.size else 0}


def check_f32(out: np.ndarray, t_exact: np.ndarray, w: np.ndarray, group_size: int):
    ref = w * t_exact
    bound = oracle_delta(group_size)
    err = np.abs(out.astype(np.float64) - ref)
    lim = bound * np.abs(ref) + 1e-38
    bad = err > lim
    assert not bad.any(), (f"{int(bad.sum())} f32 outputs outside the bound; worst rel "
                           f"{float(np.max(err / np.maximum(np.abs(ref), 1e-38))):.3e} > {bound:.3e}")
    return float(np.max(err / np.maximum(np.abs(ref), 1e-300)))


# ------------------------------------------------------------ exact decimal

_CTX = decimal.Context(prec=60)


def _dec(x: float) -> decimal.Decimal:
    return decimal.Decimal(float(x))  # exact binary value


def exact_unit(y: np.ndarray, g: np.ndarray, eps: float) -> list:
    """gated_j * (mean(gated^2) + eps)^(-1/2) for one group, at 60 digits."""
    with decimal.localcontext(_CTX):
        gated = []
        for yv, gv in zip(y.tolist(), g.tolist()):
            gd = _dec(gv)
            silu = gd / (1 + (-gd).exp())
            gated.append(_dec(yv) * silu)
        m = sum(a * a for a in gated) / len(gated) + _dec(np.float32(eps))
        nf = 1 / m.sqrt()
        return [a * nf for a in gated]


def exact_t(yd: np.ndarray, gd: np.ndarray, group_size: int, eps: float) -> np.ndarray:
    rows, width = yd.shape
    out = np.empty((rows, width), dtype=np.float64)
    for n in range(rows):
        for c0 in range(0, width, group_size):
            vals = exact_unit(yd[n, c0:c0 + group_size], gd[n, c0:c0 + group_size], eps)
            out[n, c0:c0 + group_size] = [float(v) for v in vals]
    return out
