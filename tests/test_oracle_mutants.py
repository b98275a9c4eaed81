"""The pins have teeth: each plausible mistake, planted in a copy of the
oracle's C source and built on the CPU, must make at least one pin fail.

Mutants that cannot change any result (for example widening the clamp to
-128, which no finite input reaches because |x/scale| <= 127 * (1 + 2^-24))
are deliberately not listed: no test could tell them apart.
"""
from __future__ import annotations

import pytest

import oracle
from oracle import build as obuild
from tests import pins

MUTANTS = {
    "divisor_128": ("float s = amax / 127.0f;", "float s = amax / 128.0f;"),
    "round_half_away": ("float r = nearbyintf(v);", "float r = roundf(v);"),
    "reciprocal_multiply": (
        "float v = orc_bf16_to_f32(x[k]) / s;",
        "float v = orc_bf16_to_f32(x[k]) * (127.0f / amax);"),
    "max_not_absmax": ("float a = fabsf(v);", "float a = v;"),
    "zero_row_scale_one": ("*sa = 0.0f;", "*sa = 1.0f;"),
    "reversed_k_index": (
        "s += (int64_t)a[k] * (int64_t)w[k];",
        "s += (int64_t)a[k] * (int64_t)w[K - 1 - k];"),
    "dropped_bias": (
        "if (bias) t = t + orc_bf16_to_f32(bias[n]);", "(void)bias;"),
    "bias_after_rounding": (
        "if (bias) t = t + orc_bf16_to_f32(bias[n]);",
        "if (bias) t = orc_bf16_to_f32(orc_f32_to_bf16(t))"
        " + orc_bf16_to_f32(bias[n]);"),
    "scale_product_first": (
        "t = t * sa;\n  t = t * sw;", "t = t * (sa * sw);"),
    "wrong_scale_index": (
        "float t = epi_one(acc[m * N + n], sa[m], sw[n], bias, n);",
        "float t = epi_one(acc[m * N + n], sa[m], sw[m % N], bias, n);"),
    "linear_first_scale_only": (
        "orc_f32_to_bf16(epi_one(acc, sa, sw[n], bias, n))",
        "orc_f32_to_bf16(epi_one(acc, sa, sw[0], bias, n))"),
    "bf16_round_half_up": ("u += 0x7FFFu + lsb;", "u += 0x8000u + 0 * lsb;"),
    "bf16_truncate": ("u += 0x7FFFu + lsb;", "u += 0 * lsb;"),
    "bf16_f64_no_subnormal_floor": ("if (e < -126) e = -126;", ""),
    "silu_sign": ("v / (1.0 + exp(-v))", "v / (1.0 + exp(v))"),
    "pow2_off_by_one": ("int e = ex - 1;", "int e = ex;"),
    "weight_zero_row_scale_zero": ("      sw[n] = 1.0f;", "      sw[n] = 0.0f;"),
    "scales_zero_allowed": (
        "if (!(isfinite(sw[n]) && sw[n] > 0.0f)) ++count;",
        "if (!(isfinite(sw[n]) && sw[n] >= 0.0f)) ++count;"),
    "scales_nan_allowed": (
        "if (!(isfinite(sw[n]) && sw[n] > 0.0f)) ++count;",
        "if (isinf(sw[n]) || sw[n] <= 0.0f) ++count;"),
    "swiglu_halves_swapped": (
        "const uint16_t *up = gate + F;",
        "const uint16_t *up = gate; gate = gate + F;"),
    "swiglu_unrounded_silu": (
        "double s = (double)orc_bf16_to_f32(orc_f64_to_bf16(g / (1.0 + exp(-g))));",
        "double s = g / (1.0 + exp(-g));"),
}


@pytest.fixture(scope="module")
def source():
    return obuild.SRC.read_text()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation site of {name} not unique"
    src = tmp_path / f"mut_{name}.c"
    src.write_text(source.replace(old, new))
    lib = obuild.build_from(src, tmp_path / f"libmut_{name}.so")
    orc = oracle.Oracle(lib)
    failed = []
    for check in pins.ALL_CHECKS:
        try:
            check(orc)
        except (AssertionError, oracle.OracleError):
            failed.append(check.__name__)
            break
    assert failed, f"no pin catches mutant {name}"
