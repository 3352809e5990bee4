"""Planted mistakes in the oracle are caught by its pins (CPU only).

Each case below replaces one step of the oracle with a plausible mistake (a
dropped term, a wrong sign or index, a swapped operand, a different rounding
or a different reading of the pages) and runs the pins of
``test_oracle_pins.py`` that concern that step.  At least one of them must
fail; a mutant that passes every pin would mean the oracle is not pinned
against that mistake.  Mistakes are planted in the oracle only, on the CPU.
"""
import math

import numpy as np
import pytest

from oracle import icl, numerics
from tests import test_oracle_pins as pins

_orig_attention_rows = icl.attention_rows
_orig_gate_factor = icl.gate_factor
_orig_fp8_scale = icl.fp8_scale
_orig_e4m3_round = numerics.e4m3_round
_orig_qhat = icl.OracleCache.qhat
_orig_vhat = icl.OracleCache.vhat
_orig_amax_rows = icl.amax_rows


def _attention_no_tau(q, k, v, tau):
    return _orig_attention_rows(q, k, v, 1.0)


def _attention_wrong_sign(q, k, v, tau):
    return _orig_attention_rows(q, k, v, -tau)


def _attention_wrong_axis(q, k, v, tau):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    z = (q @ k.T) * tau
    z -= z.max(axis=1, keepdims=True)
    p = np.exp(z)
    return (p @ np.asarray(v, np.float64)) / p.sum(axis=0, keepdims=True).sum()


def _gate_one_minus_tanh(gate):
    t = np.tanh(np.asarray(gate, dtype=np.float16).astype(np.float64)).astype(np.float16)
    return (np.float32(1.0) - t.astype(np.float32)).astype(np.float16)


def _gate_additive_order(gate):
    # 1 + tanh without rounding tanh to fp16 first
    return (1.0 + np.tanh(np.asarray(gate, dtype=np.float16).astype(np.float64))).astype(np.float16)


_orig_scale_queries = icl.scale_queries


def _scale_queries_one_rounding(q, mode, k_h, gate=None):
    # q * fp16(k_h * u) instead of fp16(fp16(q * k_h) * u)
    if mode != icl.SCALE_GATED_LOG:
        return _orig_scale_queries(q, mode, k_h, gate)
    kh = np.asarray(k_h, dtype=np.float16).astype(np.float32)[:, None]
    u = icl.gate_factor(gate).astype(np.float32)[..., None]
    f = (kh * u).astype(np.float16).astype(np.float32)
    return (np.asarray(q, np.float16).astype(np.float32) * f).astype(np.float16)


def _fp8_scale_swapped(amax):
    s, inv = _orig_fp8_scale(amax)
    return inv, s


def _fp8_scale_divides_by_256(amax):
    a = np.float32(amax)
    if a == 0:
        return np.float32(1.0), np.float32(1.0)
    return np.float32(a / np.float32(256)), np.float32(np.float32(256) / a)


def _e4m3_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(a > 448):
        raise ValueError("unclamped")
    _, E = np.frexp(a)
    e = np.maximum(E - 1, -6)
    spacing = np.ldexp(1.0, e - 3)
    return np.copysign(np.floor(a / spacing + 0.5) * spacing, x)


def _e4m3_two_mantissa_bits(x):
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(a > 448):
        raise ValueError("unclamped")
    _, E = np.frexp(a)
    e = np.maximum(E - 1, -6)
    spacing = np.ldexp(1.0, e - 2)
    return np.copysign(np.round(a / spacing) * spacing, x)


def _length_log2(n):
    return np.float32(math.log2(max(int(n), 1)))


def _length_unclamped_plus_one(n):
    return np.float32(math.log(int(n) + 1))


def _qhat_uses_k_scale(self, qt, b, h):
    x = qt[:, h, :]
    if self.precision == icl.PREC_FP8_E4M3:
        return icl.quantize(x, self.inv[1, b, h]) * np.float64(self.scales[1, b, h])
    return x.astype(np.float64)


def _qhat_not_quantised(self, qt, b, h):
    return qt[:, h, :].astype(np.float64)


def _qhat_own_rows_scale(self, qt, b, h):
    # the query rows' own amax instead of the context's scale
    x = qt[:, h, :]
    if self.precision == icl.PREC_FP8_E4M3:
        s, inv = icl.fp8_scale(float(np.max(np.abs(x.astype(np.float64)))))
        return icl.quantize(x, inv) * np.float64(s)
    return x.astype(np.float64)


def _vhat_uses_k_scale(self, b, h):
    if self.precision == icl.PREC_FP8_E4M3:
        return numerics.E4M3_VALUES[self.v_codes_b[b][h]] * np.float64(self.scales[1, b, h])
    return self.v16[b][:, h, :].astype(np.float64)


def _amax_over_d_only_first_row(x):
    return np.max(np.abs(np.asarray(x, dtype=np.float64)[:1]), axis=(0, 2))


def _head_factors_not_fp16(L32, coef):
    # the per-head factor left in float32 (no conversion to fp16)
    return np.float32(L32) * np.asarray(coef, dtype=np.float32)


# (name, target object, attribute, replacement, pins that should catch it)
MUTANTS = [
    ("dropped tau", icl, "attention_rows", _attention_no_tau,
     [pins.test_attention_closed_forms, lambda: pins.test_attention_brute_force_tiny(17)]),
    ("wrong exp sign", icl, "attention_rows", _attention_wrong_sign,
     [pins.test_attention_closed_forms, lambda: pins.test_attention_brute_force_tiny(17)]),
    ("softmax normalised over the wrong axis", icl, "attention_rows", _attention_wrong_axis,
     [pins.test_attention_closed_forms, lambda: pins.test_attention_brute_force_tiny(17)]),
    ("1 - tanh in the gate", icl, "gate_factor", _gate_one_minus_tanh,
     [pins.test_scaling_worked_examples, pins.test_gate_factor_over_every_fp16_gate]),
    ("gate and head factor combined before q (q * fp16(k_h u))", icl, "scale_queries",
     _scale_queries_one_rounding,
     [pins.test_gated_scaling_equals_eager_fp16_passes]),
    ("tanh not rounded to fp16 before adding 1", icl, "gate_factor", _gate_additive_order,
     [pins.test_scaling_worked_examples, pins.test_gated_scaling_equals_eager_fp16_passes]),
    ("s and inv swapped", icl, "fp8_scale", _fp8_scale_swapped,
     [pins.test_fp8_scale_maps_amax_to_448_and_bounds_error, pins.test_fp8_is_lossless_on_grid_inputs]),
    ("amax mapped to 256 instead of 448", icl, "fp8_scale", _fp8_scale_divides_by_256,
     [pins.test_fp8_scale_maps_amax_to_448_and_bounds_error, pins.test_fp8_is_lossless_on_grid_inputs]),
    ("e4m3 ties away from zero", numerics, "e4m3_round", _e4m3_ties_away,
     [pins.test_e4m3_round_matches_torch_cast_on_all_fp16_values,
      pins.test_e4m3_ties_go_to_even_and_error_is_at_most_half_spacing]),
    ("e4m3 with two mantissa bits", numerics, "e4m3_round", _e4m3_two_mantissa_bits,
     [pins.test_e4m3_round_matches_torch_cast_on_all_fp16_values, pins.test_e4m3_code_points_match_ocp_table]),
    ("log2 instead of ln", icl, "length_scalar", _length_log2,
     [pins.test_length_scalar_closed_forms]),
    ("ln(n + 1), no clamp", icl, "length_scalar", _length_unclamped_plus_one,
     [pins.test_length_scalar_closed_forms]),
    ("head factor not converted to fp16", icl, "head_factors", _head_factors_not_fp16,
     [pins.test_head_factor_and_identity_scalings]),
    ("Q dequantised with s_k", icl.OracleCache, "qhat", _qhat_uses_k_scale,
     [pins.test_fp8_is_lossless_on_grid_inputs, pins.test_fp8_query_codes_are_the_plain_per_head_quantisation]),
    ("Q not quantised", icl.OracleCache, "qhat", _qhat_not_quantised,
     [pins.test_query_rows_use_context_q_scale]),
    ("query rows take their own Q scale", icl.OracleCache, "qhat", _qhat_own_rows_scale,
     [pins.test_query_rows_use_context_q_scale]),
    ("V dequantised with s_k", icl.OracleCache, "vhat", _vhat_uses_k_scale,
     [pins.test_fp8_is_lossless_on_grid_inputs]),
    ("amax of the first row only", icl, "amax_rows", _amax_over_d_only_first_row,
     [pins.test_amax_matches_float_maximum, pins.test_fp8_is_lossless_on_grid_inputs]),
]


@pytest.mark.parametrize("name,target,attr,repl,checks", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(monkeypatch, name, target, attr, repl, checks):
    monkeypatch.setattr(target, attr, repl)
    failed = []
    for check in checks:
        try:
            with np.errstate(all="ignore"):
                check()
        except (AssertionError, ValueError, FloatingPointError, IndexError, TypeError) as e:
            failed.append(type(e).__name__)
    assert failed, f"mutant '{name}' passes every pin it should fail"


def test_unmutated_oracle_passes_the_same_pins():
    """The pins used above pass on the oracle as written (so each mutant's
    failure comes from the mutant)."""
    seen = set()
    for _, _, _, _, checks in MUTANTS:
        for check in checks:
            if id(check) in seen:
                continue
            seen.add(id(check))
            check()
