"""Planted mistakes in the oracle (on the CPU) must each be caught by some pin.

Every mutation below is a plausible slip in the oracle (a dropped term, a wrong sign, a
transposed operand, a wrong index or pairing).  The mutation is applied with monkeypatch
to the oracle module only; the pins of test_oracle_pins / test_oracle_golden are then run
and at least one of them must fail.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import triattention as T

import test_oracle_golden as golden
import test_oracle_pins as pins

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _pin_calls():
    calls = []
    for layout in ("half", "interleaved"):
        for d, base, qpos, offs in [(128, 1e4, 2047, [1, 2, 4, 8, 16]), (16, 500.0, 37, [1, 3, 9])]:
            calls.append(lambda layout=layout, d=d, base=base, qpos=qpos, offs=offs:
                         pins.test_p1_exact_centre_identity(layout, d, base, qpos, offs))
        calls.append(lambda layout=layout: pins.test_p2_zero_centre_is_pure_norm(layout))
        calls.append(lambda layout=layout: pins.test_p9_rope_apply_is_textbook_rope(layout))
        calls.append(lambda layout=layout: pins.test_p9_post_rope_keys_score_like_pre_rope_keys(layout, "max"))
        calls.append(lambda layout=layout: pins.test_p9_post_rope_exact_centre_identity(layout))
        calls.append(lambda layout=layout: pins.test_p6_identical_samples(layout))
    calls += [
        pins.test_p2_partial_concentration_norm_coefficient,
        pins.test_p3_theta_hand_values,
        lambda: pins.test_p3_single_band_345(7),
        pins.test_p3_zero_distance_quarter_turn,
        pins.test_p3_offsets_are_averaged,
        pins.test_p4_shift_invariance,
        pins.test_p4_key_scaling,
        pins.test_p4_mean_fold_linearity,
        pins.test_p4_identical_heads_and_max,
        pins.test_p4_zero_key_scores_zero,
        pins.test_p4_r_above_one_not_clamped,
        pins.test_p5_edge_cases,
        pins.test_p6_rotating_samples_have_zero_centre,
        pins.test_p6_scaling_and_permutation,
        pins.test_p7_dense_rows_are_bit_copies,
        pins.test_p7_paged_forward_packing,
        pins.test_p10_fp8_e4m3_values_fixed_by_the_format,
        pins.test_p10_bf16_values_fixed_by_the_format,
        pins.test_p10_bf16_all_patterns_match_torch,
        pins.test_p10_stored_keys_decode_with_their_scale,
        pins.test_p11_hand_value_two_bands,
        pins.test_p12_one_key_returns_its_value,
        pins.test_p12_equal_logits_average_the_values,
        pins.test_p11_band_magnitudes_enter_only_through_the_key_norm,
    ]
    for layout in ("half", "interleaved"):
        calls.append(lambda layout=layout: pins.test_p11_aligned_phases_closed_form(layout))
        calls.append(lambda layout=layout: pins.test_p11_single_band_centre_matches_amplitude_series(layout))
        calls.append(lambda layout=layout: pins.test_p12_hand_weighting_three_to_one(layout))
        calls.append(lambda layout=layout: pins.test_p12_relative_positions_and_post_rope_keys(layout))
    calls += [
        pins.test_p13_kv_head_reads_its_contiguous_query_heads,
        pins.test_p13_score_of_kv_head_one_hand_value,
        pins.test_p13_bound_hand_values_two_heads,
        pins.test_p13_band_without_query_energy_adds_nothing,
    ]
    for layout in ("half", "interleaved"):
        for reduce in ("max", "mean"):
            calls.append(lambda layout=layout, reduce=reduce:
                         pins.test_p13_bound_is_reached_by_aligned_phases(layout, reduce))
    calls += [lambda t=t: pins.test_p5_select_matches_brute_force(t) for t in range(60)]
    with open(golden.GOLDEN) as fh:
        import json
        for case in json.load(fh)["cases"]:
            calls.append(lambda case=case: golden.test_printed_memory_ratios(case))
    return calls


def _some_pin_fails():
    for call in _pin_calls():
        try:
            call()
        except (AssertionError, ValueError, IndexError):
            return True
    return False


# ---- mutated pieces (each plants one mistake) ------------------------------------------

def _theta_wrong_exponent(base, head_dim):
    f = np.arange(head_dim // 2, dtype=np.float64)
    return np.float64(base) ** (-1.0 * f / head_dim)


def _bands_swapped(x, layout="half"):
    other = {"half": "interleaved", "interleaved": "half"}[layout]
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if other == "half":
        return x[..., : d // 2] + 1j * x[..., d // 2:]
    return x[..., 0::2] + 1j * x[..., 1::2]


def _bands_conjugated(x, layout="half"):
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if layout == "half":
        return x[..., : d // 2] - 1j * x[..., d // 2:]
    return x[..., 0::2] - 1j * x[..., 1::2]


def _trig(kind):
    def trig(k_bands, key_pos, query_pos, center_h, theta, offsets):
        q_abs = np.abs(center_h)
        q_arg = np.arctan2(center_h.imag, center_h.real)
        if kind == "atan2_transposed":
            q_arg = np.arctan2(center_h.real, center_h.imag)
        k_abs = np.abs(k_bands)
        k_arg = np.arctan2(k_bands.imag, k_bands.real)
        total = np.zeros(k_bands.shape[0])
        for delta in offsets:
            if kind == "distance_sign":
                dist = key_pos.astype(float) - query_pos - delta
            elif kind == "offset_dropped":
                dist = query_pos - key_pos.astype(float)
            else:
                dist = query_pos - key_pos.astype(float) + delta
            phase = dist[:, None] * theta[None, :] + q_arg[None, :] - k_arg
            if kind == "arg_sign":
                phase = dist[:, None] * theta[None, :] - q_arg[None, :] + k_arg
            total += np.sum(q_abs[None, :] * k_abs * np.cos(phase), axis=1)
        if kind == "sum_not_mean":
            return total
        return total / len(offsets)
    return trig


def _norm(kind):
    def norm(k_bands, center_h, mean_abs_h):
        R = T.concentration(center_h, mean_abs_h)
        if kind == "dropped":
            return np.zeros(k_bands.shape[0])
        coef = (R if kind == "R_not_1mR" else 1.0 - R) * mean_abs_h
        if kind == "no_mean_abs":
            coef = 1.0 - R
        return np.sum(coef[None, :] * np.abs(k_bands), axis=1)
    return norm


def _select(kind):
    orig = T.select_top_b

    def sel(scores, length, budget, window):
        L = int(length)
        if L <= budget:
            return np.arange(L)
        w = min(window, budget)
        if kind == "window_not_forced":
            w = 0
        n_cand = L - w
        s = np.asarray(scores, dtype=float)[:n_cand].copy()
        s[np.isnan(s)] = -np.inf
        slots = np.arange(n_cand)
        if kind == "ties_high_slot":
            order = np.lexsort((-slots, -s))
        elif kind == "ascending_scores":
            order = np.lexsort((slots, s))
        else:
            order = np.lexsort((slots, -s))
        take = budget - w
        if kind == "off_by_one":
            take -= 1
        top = slots[order[:take]]
        return np.sort(np.concatenate([top, np.arange(n_cand, L)]))
    return sel if kind else orig


_rope_apply = T.rope_apply


def _rope_inverse_ignored(x, positions, *, base, layout="half", inverse=False):
    return _rope_apply(x, positions, base=base, layout=layout, inverse=False)


def _rope_sin_sign(x, positions, *, base, layout="half", inverse=False):
    return _rope_apply(x, -np.asarray(positions), base=base, layout=layout, inverse=inverse)


def _fp8_bias_8(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    out = T.__dict__["_orig_decode_fp8"](c) / 2.0
    out[(c & 0x78) == 0] *= 2.0          # subnormals unchanged, normals off by the bias
    return out


def _fp8_no_subnormals(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    out = T.__dict__["_orig_decode_fp8"](c)
    out[(c & 0x78) == 0] = 0.0
    return out


def _bf16_bias_126(bits):
    # slip: exponent bias off by one
    return T.__dict__["_orig_decode_bf16"](bits) * 2.0


def _bf16_mantissa_8bit(bits):
    # slip: the 7-bit mantissa read as if it had 8 bits
    b = np.asarray(bits).astype(np.int64) & 0xFFFF
    e = (b >> 7) & 0xFF
    m = (b & 0x7F).astype(np.float64)
    val = np.where(e == 0, m * 2.0 ** -133, (1.0 + m / 256.0) * np.exp2(e - 127.0))
    return np.where(b & 0x8000, -1.0, 1.0) * val


def _stored_scale_divided(raw, dtype, scale=1.0):
    # slip: the head's scale divides instead of multiplying
    return T.__dict__["_orig_decode_stored"](raw, dtype, 1.0 / scale)


def _calib_abs_of_mean(q, layout="half"):
    qb = T.split_bands(q, layout)
    c = qb.mean(axis=0)
    return c, np.abs(c)


def _compact_freed_off_by_one(pool_k, pool_v, bt, length, kept_by_unit, page=16):
    out = T.__dict__["_orig_compact"](pool_k, pool_v, bt, length, kept_by_unit, page)
    k, v, freed, new_len = out
    return k, v, freed[1:], new_len


def _unit_series_amplitude_kept(k_bands, key_pos, query_pos, center_h, theta, offsets):
    # slip: the key magnitudes stay inside the phase-only series
    out = T.__dict__["_orig_unit"](k_bands, key_pos, query_pos, center_h, theta, offsets)
    return out * np.sqrt(np.sum(np.abs(k_bands) ** 2, axis=1)) / np.sqrt(k_bands.shape[1])


def _unit_series_phase_sign(k_bands, key_pos, query_pos, center_h, theta, offsets):
    # slip: the key's phase enters with the wrong sign
    return T.__dict__["_orig_unit"](np.conj(k_bands), key_pos, query_pos, center_h, theta, offsets)


def _attention_key_not_rotated(q, keys, values, *, base, key_pos, query_pos, layout="half", key_space="pre"):
    # slip: the kept keys are used without RoPE at their positions
    return T.__dict__["_orig_attn"](q, keys, values, base=base, key_pos=key_pos, query_pos=query_pos,
                                     layout=layout, key_space="post")


def _attention_no_scale(q, keys, values, *, base, key_pos, query_pos, layout="half", key_space="pre"):
    # slip: logits not divided by sqrt(d)
    return T.__dict__["_orig_attn"](np.asarray(q, dtype=np.float64) * np.sqrt(np.asarray(q).shape[-1]), keys,
                                     values, base=base, key_pos=key_pos, query_pos=query_pos, layout=layout,
                                     key_space=key_space)


def _l2_as_l1(bands):
    # slip: the norm of the vector taken as the sum of band magnitudes
    return np.sum(np.abs(bands), axis=-1)


def _unit_heads_strided(center, mean_abs, layer, kv_head, group):
    # slip: query heads of a KV head taken with a stride of n_kvh instead of contiguously
    n_qh = np.asarray(mean_abs).shape[1]
    hs = slice(kv_head, None, n_qh // group)
    return T._as_complex(np.asarray(center)[layer, hs]), np.asarray(mean_abs, np.float64)[layer, hs]


def _unit_heads_offset(center, mean_abs, layer, kv_head, group):
    # slip: the group starts one KV head late
    n_qh = np.asarray(mean_abs).shape[1]
    k = min(kv_head + 1, n_qh // group - 1)
    hs = slice(k * group, (k + 1) * group)
    return T._as_complex(np.asarray(center)[layer, hs]), np.asarray(mean_abs, np.float64)[layer, hs]


def _bound(kind):
    def bound(keys, center, mean_abs, *, layout="half", reduce="max", form="additive"):
        if form != "additive":
            return T.__dict__["_orig_bound"](keys, center, mean_abs, layout=layout, reduce=reduce, form=form)
        center = T._as_complex(center)
        mean_abs = np.asarray(mean_abs, dtype=np.float64)
        if center.ndim == 1:
            center, mean_abs = center[None, :], mean_abs[None, :]
        k_abs = np.abs(T.split_bands(np.asarray(keys, dtype=np.float64), layout))
        heads = []
        for h in range(center.shape[0]):
            R = T.concentration(center[h], mean_abs[h])
            if kind == "abs_dropped":
                coef = np.abs(center[h]) + (1.0 - R) * mean_abs[h]
            elif kind == "no_centre_term":
                coef = np.abs((1.0 - R) * mean_abs[h])
            else:
                coef = np.abs(center[h]) + np.abs((1.0 - R) * mean_abs[h])
            heads.append(np.sum(coef[None, :] * k_abs, axis=1))
        heads = np.stack(heads, axis=0)
        if kind == "summed_over_heads":
            return heads.sum(axis=0)
        if kind == "inflated":
            return 2.0 * T._reduce_heads(heads, reduce)
        return T._reduce_heads(heads, reduce)
    return bound


def _concentration(zero_over_zero):
    def conc(center, mean_abs):
        center = np.asarray(center, dtype=np.complex128)
        mean_abs = np.asarray(mean_abs, dtype=np.float64)
        with np.errstate(divide="ignore", invalid="ignore"):
            out = np.abs(center) / mean_abs
        out[mean_abs == 0] = zero_over_zero
        return out
    return conc


MUTATIONS = {
    "theta_exponent": ("rope_theta", _theta_wrong_exponent),
    "bands_pairing": ("split_bands", _bands_swapped),
    "bands_conjugated": ("split_bands", _bands_conjugated),
    "distance_sign": ("_trig_term", _trig("distance_sign")),
    "offset_dropped": ("_trig_term", _trig("offset_dropped")),
    "arg_sign": ("_trig_term", _trig("arg_sign")),
    "atan2_transposed": ("_trig_term", _trig("atan2_transposed")),
    "sum_not_mean": ("_trig_term", _trig("sum_not_mean")),
    "norm_dropped": ("_norm_term", _norm("dropped")),
    "norm_R_not_1mR": ("_norm_term", _norm("R_not_1mR")),
    "norm_no_mean_abs": ("_norm_term", _norm("no_mean_abs")),
    "select_window_not_forced": ("select_top_b", _select("window_not_forced")),
    "select_ties_high_slot": ("select_top_b", _select("ties_high_slot")),
    "select_ascending": ("select_top_b", _select("ascending_scores")),
    "select_off_by_one": ("select_top_b", _select("off_by_one")),
    "calibrate_abs_of_mean": ("calibrate", _calib_abs_of_mean),
    "compact_freed_off_by_one": ("compact_paged_sequence", _compact_freed_off_by_one),
    "rope_inverse_ignored": ("rope_apply", _rope_inverse_ignored),
    "rope_angle_sign": ("rope_apply", _rope_sin_sign),
    "fp8_exponent_bias": ("decode_fp8_e4m3", _fp8_bias_8),
    "fp8_no_subnormals": ("decode_fp8_e4m3", _fp8_no_subnormals),
    "mult_amplitude_kept": ("_trig_unit_term", _unit_series_amplitude_kept),
    "mult_phase_sign": ("_trig_unit_term", _unit_series_phase_sign),
    "mult_norm_l1": ("_l2_norm", _l2_as_l1),
    "attention_key_not_rotated": ("decode_attention", _attention_key_not_rotated),
    "attention_no_scale": ("decode_attention", _attention_no_scale),
    "bf16_exponent_bias": ("decode_bf16", _bf16_bias_126),
    "bf16_mantissa_width": ("decode_bf16", _bf16_mantissa_8bit),
    "stored_scale_divided": ("decode_stored", _stored_scale_divided),
    "gqa_strided_heads": ("unit_heads", _unit_heads_strided),
    "gqa_group_offset": ("unit_heads", _unit_heads_offset),
    "bound_abs_dropped": ("score_magnitude_bound", _bound("abs_dropped")),
    "bound_summed_over_heads": ("score_magnitude_bound", _bound("summed_over_heads")),
    "bound_inflated": ("score_magnitude_bound", _bound("inflated")),
    "bound_no_centre_term": ("score_magnitude_bound", _bound("no_centre_term")),
    "concentration_0_over_0_is_1": ("concentration", _concentration(1.0)),
    "concentration_0_over_0_is_nan": ("concentration", _concentration(np.nan)),
}


def test_unmutated_oracle_passes_every_pin():
    assert not _some_pin_fails()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, repl = MUTATIONS[name]
    monkeypatch.setitem(T.__dict__, "_orig_compact", T.compact_paged_sequence)
    monkeypatch.setitem(T.__dict__, "_orig_decode_fp8", T.decode_fp8_e4m3)
    monkeypatch.setitem(T.__dict__, "_orig_unit", T._trig_unit_term)
    monkeypatch.setitem(T.__dict__, "_orig_attn", T.decode_attention)
    monkeypatch.setitem(T.__dict__, "_orig_bound", T.score_magnitude_bound)
    monkeypatch.setitem(T.__dict__, "_orig_decode_bf16", T.decode_bf16)
    monkeypatch.setitem(T.__dict__, "_orig_decode_stored", T.decode_stored)
    monkeypatch.setattr(T, attr, repl)
    if hasattr(oracle, attr):
        monkeypatch.setattr(oracle, attr, repl)
    assert _some_pin_fails(), f"planted mistake {name!r} was not caught by any pin"
