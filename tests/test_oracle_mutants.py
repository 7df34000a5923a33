"""The pins have teeth: plausible mistakes planted in copies of the oracle
(on the CPU, in a temporary directory) must each fail at least one pin.

Each mutant is the oracle's C source with one textual change, compiled with
the oracle's own flags and loaded through a fresh copy of the oracle's
Python wrapper; then the pin tests run against it.
"""
import importlib.util
import os
import subprocess

import pytest

import test_oracle_casts as casts
import test_oracle_nbg as nbg
import test_oracle_pins as pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ggrms_oracle.c")
INIT = os.path.join(ROOT, "oracle", "__init__.py")

MUTANTS = {
    "eps_before_mean": ("m2 / (float)G + eps", "(m2 + eps) / (float)G"),
    "eps_outside_root": ("1.0f / sqrtf(m2 / (float)G + eps)", "1.0f / sqrtf(m2 / (float)G) + eps"),
    "divisor_off_by_one": ("m2 / (float)G", "m2 / (float)(G + 1)"),
    "silu_sign": ("return x / (1.0f + expf(-x));", "return x / (1.0f + expf(x));"),
    "sigmoid_not_silu": ("return x / (1.0f + expf(-x));", "return 1.0f / (1.0f + expf(-x));"),
    "no_intermediate_cast": ("if (ri) t = round_trip(t, dtype);", "(void)ri;"),
    "always_intermediate_cast": ("if (ri) t = round_trip(t, dtype);", "t = round_trip(t, dtype == GGRMS_ORACLE_F32 ? GGRMS_ORACLE_BF16 : dtype);"),
    "intermediate_cast_wrong_type": ("if (ri) t = round_trip(t, dtype);", "if (ri) t = round_trip(t, GGRMS_ORACLE_BF16);"),
    "weight_index": ("norm_weight + (per_group ? 0 : col0)", "norm_weight"),
    "sum_not_squared": ("m2 = m2 + a[j] * a[j]", "m2 = m2 + fabsf(a[j])"),
    "gate_uses_y_stride": ("n * gate_row_stride + col0", "n * y_row_stride + col0"),
    "y_and_gate_swapped": ("yf * ggrms_oracle_silu(load_elem(gate, goff + j, dtype));",
                           "load_elem(gate, goff + j, dtype) * ggrms_oracle_silu(yf);"),
    "nbg_reduces_gated": ("norm_first ? yf :",
                          "norm_first ? yf * ggrms_oracle_silu(load_elem(gate, goff + j, dtype)) :"),
    "nbg_drops_gate": ("            t = t * ggrms_oracle_silu(load_elem(gate, goff + j, dtype));\n", ""),
    "nbg_weight_index": ("t = t * w[j];", "t = t * w[0];"),
    "nbg_silu_of_y": ("            t = t * ggrms_oracle_silu(load_elem(gate, goff + j, dtype));",
                      "            t = t * ggrms_oracle_silu(load_elem(y, yoff + j, dtype));"),
    "ties_away_from_zero": ("(frac == 0.5f && fmodf(k, 2.0f) != 0.0f)", "frac == 0.5f"),
    "truncating_cast": ("if (frac > 0.5f || (frac == 0.5f && fmodf(k, 2.0f) != 0.0f)) k += 1.0f;", ""),
    "flush_subnormals": ("if (lead < emin) lead = emin;", "if (lead < emin) return copysignf(0.0f, x);"),
    "f16_widen_bias": ("(int)expo - 25", "(int)expo - 24"),
    "bf16_nan_to_inf": ("return (uint16_t)(sign | 0x7FC0u);", "return (uint16_t)(sign | 0x7F80u);"),
    "f16_overflow_saturates": ("if (r > F16_MAX) return (uint16_t)(sign | 0x7C00u);", "if (r > F16_MAX) return (uint16_t)(sign | 0x7BFFu);"),
}

PIN_CALLS = [
    lambda m: pins.test_matches_fp64_chain(m, 4, 64, 4, pins.F32, 0),
    lambda m: pins.test_matches_fp64_chain(m, 4, 100, 6, pins.F16, 1),
    lambda m: pins.test_matches_fp64_chain(m, 2, 960, 2, pins.BF16, 1),
    lambda m: pins.test_matches_fp64_chain(m, 2, 65, 3, pins.BF16, 0),
    lambda m: pins.test_eps_dominated_groups(m, pins.F32, 0),
    lambda m: pins.test_wide_dynamic_range(m, pins.F16),
    lambda m: pins.test_strided_views(m, pins.F16),
    lambda m: pins.test_matches_exact_decimal(m, 5, pins.F32, 0),
    lambda m: pins.test_golden_closed_form_cases(m),
    lambda m: pins.test_silu_closed_forms(m),
    lambda m: pins.test_special_values(m),
    lambda m: casts.test_round_matches_ieee_definition(m, casts.BF16),
    lambda m: casts.test_round_matches_ieee_definition(m, casts.F16),
    lambda m: casts.test_widen_exhaustive(m, casts.F16),
    lambda m: casts.test_widen_exhaustive(m, casts.BF16),
    lambda m: casts.test_round_special_values(m, casts.BF16),
    lambda m: casts.test_round_special_values(m, casts.F16),
    lambda m: nbg.test_nbg_matches_fp64_chain(m, 3, 64, 3, nbg.F32, False),
    lambda m: nbg.test_nbg_matches_fp64_chain(m, 2, 128, 4, nbg.F16, True),
    lambda m: nbg.test_per_group_weight_gate_first(m, nbg.BF16, 1),
]


def _load_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    mdir = tmp_path / name
    mdir.mkdir()
    (mdir / "ggrms_oracle.c").write_text(src.replace(old, new))
    (mdir / "ggrms_oracle.h").write_text(open(os.path.join(ROOT, "oracle", "ggrms_oracle.h")).read())
    spec = importlib.util.spec_from_file_location(f"oracle_mutant_{name}", INIT)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    so = str(mdir / "libmutant.so")
    subprocess.run(["gcc", *mod.CFLAGS, "-o", so, str(mdir / "ggrms_oracle.c"), "-lm"], check=True)
    mod._LIB = so
    mod._lib = None
    return mod


def test_unmutated_oracle_passes_the_subset(oracle_mod):
    for call in PIN_CALLS:
        call(oracle_mod)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    mod = _load_mutant(tmp_path, name, old, new)
    caught = []
    for i, call in enumerate(PIN_CALLS):
        try:
            call(mod)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(i)
    assert caught, f"mutant {name} passed every pin"
