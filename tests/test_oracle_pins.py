"""Pins for the oracle's whole operation (CPU only).

Each test holds the oracle to something other than itself:
  * the unfused op chain the "gated_group_rmsnorm" page's intro names,
    built from library routines (torch silu and rms_norm) in float64, with
    the page's casts applied by torch's casts -- bit-exact wherever the
    rounding is not within the oracle's f32 error of a tie;
  * the page's formula at 60 decimal digits (Python decimal) on tiny inputs;
  * closed forms (G = 1, silu(0), silu(32) = 32, hand-derived cases in
    tests/golden/closed_form_cases.json);
  * invariants the formula implies: reduction to plain group RMSNorm when
    the gate is large, unit RMS when eps = 0, exact invariance under
    power-of-two scaling, sign symmetry, zero padding of a group, row
    permutation, and the identity of the two modes for f32 data.
"""
import json
import os

import numpy as np
import pytest
import torch

import refs

F32, F16, BF16 = 0, 1, 2
DT_IDS = {F32: "f32", F16: "f16", BF16: "bf16"}
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _gen(rows, width, dtype, seed, y_scale=1.0, g_scale=1.0, g_shift=0.0):
    """Random storage arrays (y, gate) and an f32 weight, drawn here with numpy
    and rounded by torch casts."""
    rng = np.random.default_rng(seed)
    y = rng.standard_normal((rows, width)) * y_scale
    g = rng.standard_normal((rows, width)) * g_scale + g_shift
    w = rng.uniform(0.5, 1.5, width).astype(np.float32)
    return refs.round64(y, dtype), refs.round64(g, dtype), w


def _run(oracle_mod, y, g, w, G, eps, dtype, ri):
    rows, width = y.shape
    return oracle_mod.forward_2d(y, g, w, G, eps, dtype, ri)


def _t_exact(y, g, G, eps, dtype):
    return refs.chain_fp64(refs.widen64(y, dtype), refs.widen64(g, dtype), G,
                           float(np.float32(eps)))


def _check(out, y, g, w, G, eps, dtype, ri, min_exact=0.6):
    t = _t_exact(y, g, G, eps, dtype)
    if dtype == F32:
        return refs.check_f32(out, t, w.astype(np.float64)[None, :], G)
    return refs.check_16bit(out, t, w.astype(np.float64)[None, :], G, dtype, ri, min_exact)


# ------------------------------------------------------- vs the fp64 chain

CASES = [
    # rows, G, groups
    (4, 64, 4), (3, 1, 17), (5, 2, 9), (2, 3, 11), (3, 7, 5), (2, 63, 3), (2, 65, 3),
    (4, 100, 6), (2, 127, 2), (3, 128, 4), (2, 960, 2), (1, 4096, 1),
]


@pytest.mark.parametrize("dtype", [F32, F16, BF16], ids=DT_IDS.get)
@pytest.mark.parametrize("ri", [0, 1])
@pytest.mark.parametrize("rows,G,groups", CASES)
def test_matches_fp64_chain(oracle_mod, rows, G, groups, dtype, ri):
    y, g, w = _gen(rows, G * groups, dtype, seed=G * 31 + groups + 7 * ri + dtype)
    out = _run(oracle_mod, y, g, w, G, 1e-5, dtype, ri)
    _check(out, y, g, w, G, 1e-5, dtype, ri, min_exact=0.6 if G < 4096 else 0.3)


@pytest.mark.parametrize("dtype", [F32, F16, BF16], ids=DT_IDS.get)
@pytest.mark.parametrize("ri", [0, 1])
def test_eps_dominated_groups(oracle_mod, dtype, ri):
    """Small activations, so eps is comparable to the mean of squares: a wrong
    eps placement (outside the root, scaled by G, before the mean) shows."""
    y, g, w = _gen(6, 256, dtype, seed=99, y_scale=2e-3)
    for eps in (1e-5, 1e-6, 3e-4):
        out = _run(oracle_mod, y, g, w, 64, eps, dtype, ri)
        _check(out, y, g, w, 64, eps, dtype, ri)


@pytest.mark.parametrize("dtype", [F16, BF16], ids=DT_IDS.get)
def test_wide_dynamic_range(oracle_mod, dtype):
    """Log-uniform magnitudes over many decades: intermediates of gated*nf
    fall into the fp16 subnormal range, so round_intermediate exercises
    gradual underflow."""
    rng = np.random.default_rng(5)
    rows, width, G = 8, 512, 128
    mag = 10.0 ** rng.uniform(-7, 1, (rows, width))
    y = refs.round64(mag * rng.choice([-1.0, 1.0], (rows, width)), dtype)
    g = refs.round64(rng.standard_normal((rows, width)) * 3, dtype)
    w = rng.uniform(0.5, 1.5, width).astype(np.float32)
    for ri in (0, 1):
        out = _run(oracle_mod, y, g, w, G, 1e-6, dtype, ri)
        _check(out, y, g, w, G, 1e-6, dtype, ri)
    if dtype == F16:
        t = _t_exact(y, g, G, 1e-6, dtype)
        assert (np.abs(t) < 2.0 ** -14).mean() > 0.05  # many subnormal intermediates


@pytest.mark.parametrize("dtype", [F32, F16, BF16], ids=DT_IDS.get)
def test_strided_views(oracle_mod, dtype):
    """y and gate as column slices of one fused buffer, and gate from a second
    buffer with yet another row stride; out has its own stride too.  A stride
    or offset mix-up changes the result."""
    rows, width, G, fw, gw = 5, 300, 100, 700, 333
    rng = np.random.default_rng(3)
    fused = refs.round64(rng.standard_normal((rows, fw)), dtype)
    other = refs.round64(rng.standard_normal((rows, gw)), dtype)
    w = rng.uniform(0.5, 1.5, width).astype(np.float32)
    for gbuf, gstride, goff in ((fused, fw, 350), (other, gw, 20)):
        out = oracle_mod.forward(fused.reshape(-1), gbuf.reshape(-1), w, rows=rows, width=width,
                                 group_size=G, y_row_stride=fw, gate_row_stride=gstride,
                                 out_row_stride=width + 3, eps=1e-5, dtype=dtype,
                                 round_intermediate=1, y_offset=17, gate_offset=goff)
        out = np.pad(out, (0, 3)).reshape(rows, width + 3)[:, :width]
        y = fused[:, 17:17 + width]
        g = gbuf[:, goff:goff + width]
        _check(out, y, g, w, G, 1e-5, dtype, 1)


# ------------------------------------------------------- exact decimal

@pytest.mark.parametrize("dtype", [F32, F16, BF16], ids=DT_IDS.get)
@pytest.mark.parametrize("ri", [0, 1])
@pytest.mark.parametrize("G", [1, 2, 5, 16, 33])
def test_matches_exact_decimal(oracle_mod, G, dtype, ri):
    """The page's formula at 60 significant digits (brute force, tiny inputs)."""
    y, g, w = _gen(2, 2 * G, dtype, seed=1000 + G + ri)
    out = _run(oracle_mod, y, g, w, G, 1e-5, dtype, ri)
    t = refs.exact_t(refs.widen64(y, dtype), refs.widen64(g, dtype), G, 1e-5)
    wd = w.astype(np.float64)[None, :]
    if dtype == F32:
        refs.check_f32(out, t, wd, G)
    else:
        refs.check_16bit(out, t, wd, G, dtype, ri, min_exact_fraction=0.5)


# ------------------------------------------------------- closed forms

def test_silu_closed_forms(oracle_mod):
    assert oracle_mod.lib().ggrms_oracle_silu(0.0) == 0.0
    # exp(-32) vanishes next to 1 in f32, so silu(32) is 32 exactly
    assert oracle_mod.lib().ggrms_oracle_silu(32.0) == 32.0
    x = np.linspace(-20, 20, 4001).astype(np.float32)
    s = oracle_mod.silu(x).astype(np.float64)
    exact = torch.nn.functional.silu(torch.from_numpy(x.astype(np.float64))).numpy()
    rel = np.abs(s - exact) / np.maximum(np.abs(exact), 1e-30)
    assert rel.max() < 4 * refs.U32
    # silu(x) - silu(-x) = x
    sm = oracle_mod.silu(-x).astype(np.float64)
    assert np.allclose(s - sm, x.astype(np.float64), rtol=4 * refs.U32, atol=1e-30)


def test_group_size_one_closed_form(oracle_mod):
    """G = 1: out = w * a / sqrt(a^2 + eps), a = y * silu(gate) (P3's JS
    example uses a one-element scale, the same degenerate case)."""
    y, g, w = _gen(3, 4, F32, seed=11)
    for eps in (1e-5, 0.0):
        out = _run(oracle_mod, y, g, w, 1, eps, F32, 0).astype(np.float64)
        yd, gd = y.astype(np.float64), g.astype(np.float64)
        a = yd / (1 + np.exp(-gd)) * gd
        ref = w.astype(np.float64) * a / np.sqrt(a * a + np.float32(eps))
        assert np.allclose(out, ref, rtol=24 * refs.U32, atol=0)
    # eps = 0: |out| = w up to the roundings of a*a, sqrt, 1/x and two products
    out0 = _run(oracle_mod, y, g, w, 1, 0.0, F32, 0).astype(np.float64)
    assert np.allclose(np.abs(out0), np.broadcast_to(w, out0.shape), rtol=6 * refs.U32, atol=0)


def test_golden_closed_form_cases(oracle_mod):
    with open(os.path.join(GOLDEN, "closed_form_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        y = np.array(c["y"], dtype=np.float32).reshape(c["rows"], c["width"])
        g = np.array(c["gate"], dtype=np.float32).reshape(c["rows"], c["width"])
        w = np.array(c["weight"], dtype=np.float32)
        out = _run(oracle_mod, y, g, w, c["group_size"], c["eps"], F32, 0)
        want = np.array(c["out"], dtype=np.float64).reshape(out.shape)
        assert np.allclose(out, want, rtol=c["rtol"], atol=0), c["name"]


# ------------------------------------------------------- invariants

@pytest.mark.parametrize("dtype", [F32, F16, BF16], ids=DT_IDS.get)
@pytest.mark.parametrize("ri", [0, 1])
def test_large_gate_reduces_to_group_rmsnorm(oracle_mod, dtype, ri):
    """gate = 32: silu(32) = 32 exactly, gated = 32*y exactly, and the op is
    the textbook group RMSNorm of y with eps/1024 (torch rms_norm, float64)."""
    rows, width, G = 4, 384, 96
    y, _, w = _gen(rows, width, dtype, seed=21)
    g = refs.round64(np.full((rows, width), 32.0), dtype)
    out = _run(oracle_mod, y, g, w, G, 1e-5, dtype, ri)
    yd = refs.widen64(y, dtype)
    t = torch.nn.functional.rms_norm(torch.from_numpy(yd).reshape(rows, -1, G), (G,),
                                     eps=float(np.float32(1e-5)) / 1024).reshape(rows, width)
    t = t.numpy()
    wd = w.astype(np.float64)[None, :]
    if dtype == F32:
        refs.check_f32(out, t, wd, G)
    else:
        refs.check_16bit(out, t, wd, G, dtype, ri)


def test_unit_rms_when_eps_zero(oracle_mod):
    """eps = 0, w = 1, f32: every group's mean of out^2 is 1."""
    rows, width, G = 6, 960, 160
    y, g, _ = _gen(rows, width, F32, seed=4)
    out = _run(oracle_mod, y, g, np.ones(width, np.float32), G, 0.0, F32, 0)
    ms = (out.astype(np.float64).reshape(rows, -1, G) ** 2).mean(-1)
    assert np.allclose(ms, 1.0, rtol=(G + 8) * refs.U32, atol=0)
    # |gated*nf| <= sqrt(G), since gated_j^2 <= m2
    assert np.abs(out).max() <= np.sqrt(G) * (1 + 4 * refs.U32)


@pytest.mark.parametrize("dtype", [F32, F16, BF16], ids=DT_IDS.get)
@pytest.mark.parametrize("ri", [0, 1])
def test_power_of_two_scaling_is_exact(oracle_mod, dtype, ri):
    """y -> 2^k y with eps -> 4^k eps leaves every output bit unchanged (all
    f32 steps scale exactly; sqrt is correctly rounded).  eps = 0 is the
    plain scale invariance."""
    y, g, w = _gen(4, 256, dtype, seed=8)
    yd = refs.widen64(y, dtype)
    # keep |y| well inside the normal range so every scaled y is exact
    yd = np.where(np.abs(yd) < 2.0 ** -6, 2.0 ** -6, yd)
    y = refs.round64(yd, dtype)
    for eps in (0.0, 2.0 ** -17):
        base = _run(oracle_mod, y, g, w, 64, eps, dtype, ri)
        for k in (-3, 1, 4):
            ys = refs.round64(yd * 2.0 ** k, dtype)
            assert np.array_equal(refs.widen64(ys, dtype), yd * 2.0 ** k)
            got = _run(oracle_mod, ys, g, w, 64, eps * 4.0 ** k, dtype, ri)
            assert np.array_equal(got.view(np.uint16 if dtype else np.uint32),
                                  base.view(np.uint16 if dtype else np.uint32))


def test_general_scaling_within_rounding(oracle_mod):
    """eps = 0: y -> alpha*y for any alpha > 0 changes the f32 output only by rounding."""
    y, g, w = _gen(4, 256, F32, seed=9)
    base = _run(oracle_mod, y, g, w, 64, 0.0, F32, 0).astype(np.float64)
    for alpha in (0.37, 3.1, 1e3):
        ys = (y.astype(np.float64) * alpha).astype(np.float32)
        got = _run(oracle_mod, ys, g, w, 64, 0.0, F32, 0).astype(np.float64)
        assert np.allclose(got, base, rtol=2 * refs.oracle_delta(64), atol=0)


@pytest.mark.parametrize("dtype", [F32, F16, BF16], ids=DT_IDS.get)
def test_sign_symmetry(oracle_mod, dtype):
    y, g, w = _gen(3, 320, dtype, seed=10)
    neg = (y.view(np.uint32) ^ np.uint32(0x80000000)).view(np.float32) if dtype == F32 else y ^ np.uint16(0x8000)
    for ri in (0, 1):
        a = _run(oracle_mod, y, g, w, 64, 1e-5, dtype, ri)
        b = _run(oracle_mod, neg, g, w, 64, 1e-5, dtype, ri)
        flip = np.uint32(0x80000000) if dtype == F32 else np.uint16(0x8000)
        av = a.view(np.uint32) if dtype == F32 else a
        bv = b.view(np.uint32) if dtype == F32 else b
        assert np.array_equal(av ^ flip, bv)


def test_zero_padding_a_group(oracle_mod):
    """A group of G = 100 padded with y = 0 to G' = 128 and eps' = eps*G/G':
    out_G = sqrt(G/G') * out_G' on the real columns (f32, round_intermediate
    off).  This is the group-size-not-a-multiple-of-64 case the lanes of one
    wave would pad."""
    rows, G, Gp, groups = 3, 100, 128, 4
    y, g, w = _gen(rows, G * groups, F32, seed=12)
    eps = 1e-3
    out = _run(oracle_mod, y, g, w, G, eps, F32, 0).astype(np.float64)
    yp = np.zeros((rows, Gp * groups), np.float32)
    gp = np.zeros((rows, Gp * groups), np.float32)
    wp = np.ones(Gp * groups, np.float32)
    for k in range(groups):
        yp[:, k * Gp:k * Gp + G] = y[:, k * G:(k + 1) * G]
        gp[:, k * Gp:k * Gp + G] = g[:, k * G:(k + 1) * G]
        wp[k * Gp:k * Gp + G] = w[k * G:(k + 1) * G]
    outp = _run(oracle_mod, yp, gp, wp, Gp, eps * G / Gp, F32, 0).astype(np.float64)
    real = np.concatenate([outp[:, k * Gp:k * Gp + G] for k in range(groups)], axis=1)
    assert np.allclose(out, np.sqrt(G / Gp) * real, rtol=1e-5, atol=0)
    pad = np.concatenate([outp[:, k * Gp + G:(k + 1) * Gp] for k in range(groups)], axis=1)
    assert not pad.any()


def test_row_permutation(oracle_mod):
    y, g, w = _gen(9, 192, BF16, seed=13)
    perm = np.random.default_rng(1).permutation(9)
    a = _run(oracle_mod, y, g, w, 64, 1e-5, BF16, 1)
    b = _run(oracle_mod, y[perm], g[perm], w, 64, 1e-5, BF16, 1)
    assert np.array_equal(a[perm], b)


def test_f32_modes_identical(oracle_mod):
    y, g, w = _gen(4, 256, F32, seed=14)
    a = _run(oracle_mod, y, g, w, 64, 1e-5, F32, 0)
    b = _run(oracle_mod, y, g, w, 64, 1e-5, F32, 1)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_special_values(oracle_mod):
    """IEEE propagation: NaN in a group makes the whole group NaN; an
    all-zero group gives zeros for eps > 0 and NaN for eps = 0; a huge
    negative gate gives silu = -0."""
    rows, width, G = 4, 16, 8
    y = np.ones((rows, width), np.float32)
    g = np.ones((rows, width), np.float32)
    y[0, 3] = np.nan
    y[1, :8] = 0.0
    g[2, 5] = -200.0
    w = np.ones(width, np.float32)
    out = _run(oracle_mod, y, g, w, G, 1e-5, F32, 0)
    assert np.isnan(out[0, :8]).all() and np.isfinite(out[0, 8:]).all()
    assert (out[1, :8] == 0).all()
    assert out[2, 5] == 0 and np.isfinite(out[2]).all()
    out0 = _run(oracle_mod, y, g, w, G, 0.0, F32, 0)
    assert np.isnan(out0[1, :8]).all()


def test_rejects_bad_arguments(oracle_mod):
    y = np.zeros(64, np.float32)
    with pytest.raises(ValueError):
        oracle_mod.forward(y, y, np.ones(64, np.float32), rows=1, width=64, group_size=48,
                           y_row_stride=64, gate_row_stride=64, out_row_stride=64, eps=1e-5,
                           dtype=F32, round_intermediate=0)
    out = oracle_mod.forward(y, y, np.ones(64, np.float32), rows=0, width=64, group_size=64,
                             y_row_stride=64, gate_row_stride=64, out_row_stride=64, eps=1e-5,
                             dtype=F32, round_intermediate=0)
    assert out.size == 0
