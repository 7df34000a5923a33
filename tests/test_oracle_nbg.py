"""Pins for the oracle's norm-before-gate operator and per-group weight (CPU).

The "com.microsoft.GatedRMSNorm" page (Description section) defines an
operator that takes the group's normaliser from the input alone,
nf = 1/sqrt(mean_j y_j^2 + eps), and multiplies y * nf by the weight and by
silu(gate), every intermediate in f32 and only the store narrowing; its
weight holds one value per column of a group, shared by every group (Inputs
table).  The oracle's
WEIGHT_PER_GROUP flag also applies to the gate-first operator.
"""
import numpy as np
import pytest
import torch

import refs

F32, F16, BF16 = 0, 1, 2
DT_IDS = {F32: "f32", F16: "f16", BF16: "bf16"}


def _gen(rows, width, dtype, seed, y_scale=1.0):
    rng = np.random.default_rng(seed)
    y = rng.standard_normal((rows, width)) * y_scale
    g = rng.standard_normal((rows, width)) * 2
    return refs.round64(y, dtype), refs.round64(g, dtype), rng


def _check(out, t_exact, G, dtype):
    """Only the store rounds: the oracle's f32 value is within the usual
    bound plus the two extra products of the exact one."""
    if dtype == F32:
        ref = t_exact
        bound = refs.oracle_delta(G) + 4 * refs.U32
        err = np.abs(out.astype(np.float64) - ref)
        assert (err <= bound * np.abs(ref) + 1e-38).all(), float((err / np.maximum(np.abs(ref), 1e-38)).max())
        return
    delta = refs.oracle_delta(G) + 4 * refs.U32
    exp_bits = refs.round64(t_exact, dtype)
    exact = ~refs.near_tie(t_exact, dtype, delta)
    d = refs.ulp_distance(out, exp_bits)
    assert not ((d != 0) & exact).any(), f"{int(((d != 0) & exact).sum())} mismatches off ties"
    assert d.max() <= 1
    assert exact.mean() > 0.6


@pytest.mark.parametrize("per_group", [False, True], ids=["per_column", "per_group"])
@pytest.mark.parametrize("dtype", [F32, F16, BF16], ids=DT_IDS.get)
@pytest.mark.parametrize("rows,G,groups", [(3, 64, 3), (2, 128, 4), (4, 1, 9), (2, 100, 3),
                                           (1, 960, 2), (3, 7, 5)])
def test_nbg_matches_fp64_chain(oracle_mod, rows, G, groups, dtype, per_group):
    """Against rms_norm(X) * scale * silu(gate) from torch library routines in float64."""
    width = G * groups
    y, g, rng = _gen(rows, width, dtype, seed=G + groups + 5 * dtype)
    wlen = G if per_group else width
    w = rng.uniform(0.5, 1.5, wlen).astype(np.float32)
    out = oracle_mod.forward_2d(y, g, w, G, 1e-5, dtype, 0, norm_before_gate=True,
                                weight_per_group=per_group)
    wcol = np.tile(w, groups) if per_group else w
    t = refs.chain_nbg_fp64(refs.widen64(y, dtype), refs.widen64(g, dtype),
                            wcol.astype(np.float64), G, float(np.float32(1e-5)))
    _check(out, t, G, dtype)


@pytest.mark.parametrize("dtype", [F32, F16], ids=DT_IDS.get)
def test_nbg_eps_dominated(oracle_mod, dtype):
    y, g, rng = _gen(4, 256, dtype, seed=3, y_scale=3e-3)
    w = rng.uniform(0.5, 1.5, 256).astype(np.float32)
    for eps in (1e-5, 1e-6):
        out = oracle_mod.forward_2d(y, g, w, 64, eps, dtype, 0, norm_before_gate=True)
        t = refs.chain_nbg_fp64(refs.widen64(y, dtype), refs.widen64(g, dtype),
                                w.astype(np.float64), 64, float(np.float32(eps)))
        _check(out, t, 64, dtype)


def test_nbg_exact_decimal(oracle_mod):
    """Tiny inputs at 60 digits: normalise y, then weight, then silu(gate)."""
    import decimal

    y, g, rng = _gen(2, 10, F32, seed=8)
    w = rng.uniform(0.5, 1.5, 10).astype(np.float32)
    out = oracle_mod.forward_2d(y, g, w, 5, 1e-5, F32, 0, norm_before_gate=True)
    ctx = decimal.Context(prec=60)
    with decimal.localcontext(ctx):
        D = lambda v: decimal.Decimal(float(v))
        for n in range(2):
            for c0 in (0, 5):
                xs = [D(v) for v in y[n, c0:c0 + 5]]
                m = sum(x * x for x in xs) / 5 + D(np.float32(1e-5))
                nf = 1 / m.sqrt()
                for j in range(5):
                    gv = D(g[n, c0 + j])
                    exact = xs[j] * nf * D(w[c0 + j]) * gv / (1 + (-gv).exp())
                    rel = abs(float((D(out[n, c0 + j]) - exact) / exact))
                    assert rel <= refs.oracle_delta(5) + 4 * refs.U32


def test_nbg_large_gate_is_scaled_rmsnorm(oracle_mod):
    """gate = 32: silu(32) = 32 exactly, so Y = 32 * rmsnorm(X) * w."""
    y, _, rng = _gen(3, 384, F32, seed=9)
    g = np.full(y.shape, 32.0, np.float32)
    w = rng.uniform(0.5, 1.5, 384).astype(np.float32)
    out = oracle_mod.forward_2d(y, g, w, 96, 1e-5, F32, 0, norm_before_gate=True)
    t = torch.nn.functional.rms_norm(torch.from_numpy(y.astype(np.float64)).reshape(3, 4, 96), (96,),
                                     eps=float(np.float32(1e-5))).reshape(3, 384).numpy()
    ref = 32.0 * t * w.astype(np.float64)
    assert np.allclose(out, ref, rtol=refs.oracle_delta(96) + 4 * refs.U32, atol=0)


@pytest.mark.parametrize("dtype", [F32, F16, BF16], ids=DT_IDS.get)
def test_nbg_power_of_two_scaling(oracle_mod, dtype):
    """y -> 2^k y with eps -> 4^k eps changes no output bit."""
    y, g, rng = _gen(3, 256, dtype, seed=10)
    yd = refs.widen64(y, dtype)
    yd = np.where(np.abs(yd) < 2.0 ** -6, 2.0 ** -6, yd)
    y = refs.round64(yd, dtype)
    w = rng.uniform(0.5, 1.5, 256).astype(np.float32)
    base = oracle_mod.forward_2d(y, g, w, 64, 2.0 ** -17, dtype, 0, norm_before_gate=True)
    for k in (-2, 3):
        ys = refs.round64(yd * 2.0 ** k, dtype)
        got = oracle_mod.forward_2d(ys, g, w, 64, 2.0 ** -17 * 4.0 ** k, dtype, 0,
                                    norm_before_gate=True)
        view = np.uint32 if dtype == F32 else np.uint16
        assert np.array_equal(got.view(view), base.view(view))


@pytest.mark.parametrize("dtype", [F32, BF16], ids=DT_IDS.get)
@pytest.mark.parametrize("ri", [0, 1])
def test_per_group_weight_gate_first(oracle_mod, dtype, ri):
    """The gate-first operator with a weight shared by every group equals the
    fp64 chain with that weight tiled over the groups."""
    rows, G, groups = 3, 128, 4
    y, g, rng = _gen(rows, G * groups, dtype, seed=11)
    w = rng.uniform(0.5, 1.5, G).astype(np.float32)
    out = oracle_mod.forward_2d(y, g, w, G, 1e-5, dtype, ri, weight_per_group=True)
    t = refs.chain_fp64(refs.widen64(y, dtype), refs.widen64(g, dtype), G, float(np.float32(1e-5)))
    wd = np.tile(w, groups).astype(np.float64)[None, :]
    if dtype == F32:
        refs.check_f32(out, t, wd, G)
    else:
        refs.check_16bit(out, t, wd, G, dtype, ri)


def test_nbg_rejects_intermediate_cast(oracle_mod):
    y, g, _ = _gen(1, 64, BF16, seed=1)
    with pytest.raises(ValueError):
        oracle_mod.forward_2d(y, g, np.ones(64, np.float32), 64, 1e-5, BF16, 1,
                              norm_before_gate=True)
