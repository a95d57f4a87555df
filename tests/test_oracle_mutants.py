"""Planted mistakes in the oracle are caught by its pins (CPU only).

Each case copies ``oracle/rac_oracle.c``, plants one plausible mistake by a
textual replacement (a dropped term, a wrong sign, index, exponent, scale,
mask or rounding), builds the copy into a temporary library and requires that
at least one pin fails on it. The real oracle passes every pin.
"""
import os

import pytest

import oracle
from oracle import build as oracle_build
from oracle_pins import ALL_PINS

MUTANTS = {
    "rotation_sign": ("yr[2 * i] = x0 * c - x1 * s;", "yr[2 * i] = x0 * c + x1 * s;"),
    "rotation_dropped_term": ("yr[2 * i + 1] = x0 * s + x1 * c;", "yr[2 * i + 1] = x1 * c;"),
    "rotation_direction": ("double c = cos(angle), s = sin(angle);",
                           "double c = cos(angle), s = -sin(angle);"),
    "frequency_exponent": ("exp(-((2.0 * i) / D) * log_base)", "exp(-((1.0 * i) / D) * log_base)"),
    "half_split_pairs": ("double x0 = xr[2 * i], x1 = xr[2 * i + 1];",
                         "double x0 = xr[i], x1 = xr[i + D / 2];"),
    "position_off_by_one": ("double angle = (double)pos[r] * theta;",
                            "double angle = (double)(pos[r] + 1) * theta;"),
    "scale_one_over_d": ("1.0 / sqrt((double)D)", "1.0 / (double)D"),
    "mask_strict": ("for (int64_t j = 0; j <= i; ++j) {\n                double p",
                    "for (int64_t j = 0; j < i; ++j) {\n                double p"),
    "mask_window": ("for (int64_t j = 0; j <= i; ++j) {\n                double dot",
                    "for (int64_t j = (i > 3 ? i - 3 : 0); j <= i; ++j) {\n                double dot"),
    "lse_log2": ("lse[r] = M + log(l);", "lse[r] = M + log2(l);"),
    "lse_no_max": ("lse[r] = M + log(l);", "lse[r] = log(l);"),
    "gqa_modulo": ("int64_t g = h / group;", "int64_t g = h % Hkv;"),
    "no_normalise": ("for (int d = 0; d < D; ++d) orow[d] /= l;", ""),
    "round_truncate": ("double n = nearbyint(r);", "double n = trunc(r);"),
    "round_half_up": ("double n = nearbyint(r);", "double n = floor(r + 0.5);"),
    "fp16_exponent_bias": ("(uint16_t)(((e - 1 + 15) << 10) | m)", "(uint16_t)(((e + 15) << 10) | m)"),
    "bf16_decode_shift": ("uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;"),
    "bwd_delta_sign": ("double ds = exp(s[j] - lse[row]) * (dp - delta[row]);",
                       "double ds = exp(s[j] - lse[row]) * (dp + delta[row]);"),
    "bwd_dq_no_scale": ("dqi[d] += tau * ds * kb[j * D + d];", "dqi[d] += ds * kb[j * D + d];"),
    "bwd_dk_uses_dout": ("dkj[d] += tau * ds * qi[d];", "dkj[d] += tau * ds * doi[d];"),
    "bwd_dv_uses_ds": ("dvj[d] += p * doi[d];", "dvj[d] += ds * doi[d];"),
    "bwd_key_pass_strict": ("for (int64_t i = j; i < N; ++i) {", "for (int64_t i = j + 1; i < N; ++i) {"),
    "bwd_delta_drops_p": ("dl += exp(s[j] - L) * dp;", "dl += dp;"),
    "half_rotation_sign": ("yr[i] = a * cs - b * sn;", "yr[i] = a * cs + b * sn;"),
    "half_partner_index": ("double a = xr[i], b = xr[i + half];",
                           "double a = xr[i], b = xr[half - 1 - i + half];"),
    "half_frequency_index": ("const double freq = exp(-(2.0 * i / D) * log_base);",
                             "const double freq = exp(-(2.0 * (half - 1 - i) / D) * log_base);"),
    "half_direction": ("const double cs = cos(turn), sn = sin(turn);",
                       "const double cs = cos(turn), sn = -sin(turn);"),
    "bwd_scale_one_over_d": ("pow((double)D, -0.5)", "pow((double)D, -1.0)"),
    "bwd_gqa_modulo": ("const int64_t kv_head = b * Hkv + h / group;",
                       "const int64_t kv_head = b * Hkv + h % Hkv;"),
    "alibi_scale_one_over_d": ("sqrt(1.0 / (double)D)", "(1.0 / (double)D)"),
    "alibi_sign": ("score[kpos] = inv_sqrt_d * qk - slope * distance;",
                   "score[kpos] = inv_sqrt_d * qk + slope * distance;"),
    "alibi_scaled_penalty": ("score[kpos] = inv_sqrt_d * qk - slope * distance;",
                             "score[kpos] = inv_sqrt_d * (qk - slope * distance);"),
    "alibi_slope_per_kv_head": ("const double slope = slopes[qhead];",
                                "const double slope = slopes[qhead / heads_per_kv];"),
    "alibi_distance_offset": ("const double distance = (double)(qpos - kpos);",
                              "const double distance = (double)(qpos - kpos + 1);"),
    "alibi_gqa_modulo": ("const int64_t kvh = batch * Hkv + qhead / heads_per_kv;",
                         "const int64_t kvh = batch * Hkv + qhead % Hkv;"),
    "alibi_bwd_penalty_sign": ("return slopes ? slopes[h] * (double)(i - j) : 0.0;",
                               "return slopes ? slopes[h] * (double)(j - i) : 0.0;"),
    "alibi_bwd_key_pass_drops_penalty": (
        "double p = exp(tau * dot - alibi_penalty(slopes, h, i, j) - lse[row]);",
        "double p = exp(tau * dot - lse[row]);"),
    "alibi_bwd_scaled_penalty": ("s[j] = tau * dot - alibi_penalty(slopes, h, i, j);",
                                 "s[j] = tau * (dot - alibi_penalty(slopes, h, i, j));"),
    "alibi_mask_strict": ("for (int64_t kpos = 0; kpos <= qpos; ++kpos) {\n                const double w",
                          "for (int64_t kpos = 0; kpos < qpos; ++kpos) {\n                const double w"),
}


def test_pins_pass_on_real_oracle(orc):
    for pin in ALL_PINS:
        pin(orc)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = open(oracle_build.SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, "mutation anchor must occur exactly once: %r" % old
    mutated = tmp_path / "rac_oracle_mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle_build.build(src=str(mutated), out=str(tmp_path / ("liboracle_%s.so" % name)))
    mut = oracle.Oracle(lib)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(mut)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, "no pin caught the planted mistake %r" % name
