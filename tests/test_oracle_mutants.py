"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case copies `oracle/attn_oracle.c`, plants one plausible mistake by a
textual substitution, compiles the copy with gcc into a temporary directory and
runs every pin against it.  A case passes when at least one pin fails; a pin
set that cannot see the mistake would make this test fail.  The real oracle is
never modified.
"""
import os
import shutil

import pytest

import oracle
from oracle import build as obuild
from oracle_pins import ALL_PINS

MUTANTS = [
    ("drop_scale", "s[j] = scale * dot;", "s[j] = dot;"),
    ("max_sign", "exp(s[j] - m)", "exp(m - s[j])"),
    ("no_max_in_lse", "*lse_out = m + log(l);", "*lse_out = log(l);"),
    ("no_normalisation", "o_out[d] /= l;", "o_out[d] /= 1.0;"),
    ("causal_off_by_one", "int64_t lim = i + ((int64_t)Sk - (int64_t)Sq);",
     "int64_t lim = i + ((int64_t)Sk - (int64_t)Sq) - 1;"),
    ("causal_top_left", "int64_t lim = i + ((int64_t)Sk - (int64_t)Sq);", "int64_t lim = i;"),
    ("grouped_heads_interleaved", "const int64_t kvh = h / (Hq / Hkv);",
     "const int64_t kvh = h % Hkv;"),
    ("scores_from_v", "qrow[d] * load_elem(k, dtype, kr", "qrow[d] * load_elem(v, dtype, kr"),
    ("values_from_k", "w * load_elem(v, dtype, vr", "w * load_elem(k, dtype, vr"),
    ("kv_stride_uses_sq", "(size_t)kvh) * (size_t)Sk * (size_t)D",
     "(size_t)kvh) * (size_t)Sq * (size_t)D"),
    ("empty_row_lse_zero", "*lse_out = -INFINITY;", "*lse_out = 0.0;"),
    ("fp16_bias", "expo - 25", "expo - 24"),
    ("fp16_subnormal", "ldexp((double)frac, -24)", "ldexp((double)frac, -25)"),
    ("bf16_shift", "(uint32_t)bits << 16", "(uint32_t)bits << 15"),
    ("last_key_dropped", "for (int64_t j = 0; j <= last; ++j) {\n        const double w",
     "for (int64_t j = 0; j < last; ++j) {\n        const double w"),
    ("exp_weight_unused_in_sum", "l += w;", "l += 1.0;"),
    ("bwd_drop_row_term", "const double ds = p[j] * (dp[j] - pdp);", "const double ds = p[j] * dp[j];"),
    ("bwd_dk_unscaled", "dk[koff + (size_t)d] += scale * ds * qrow[d];",
     "dk[koff + (size_t)d] += ds * qrow[d];"),
    ("bwd_dv_from_ds", "dv[koff + (size_t)d] += p[j] * grow[d];", "dv[koff + (size_t)d] += ds * grow[d];"),
    ("bwd_dq_from_v", "dqi[d] += scale * ds * load_elem(k, dtype, koff", "dqi[d] += scale * ds * load_elem(v, dtype, koff"),
    ("bwd_unnormalised", "for (int64_t j = 0; j <= last; ++j) p[j] /= l;", ""),
    ("bwd_causal_top_left", "const int64_t diag = i + ((int64_t)Sk - (int64_t)Sq);", "const int64_t diag = i;"),
    ("bwd_dp_from_q", "dot += grow[d] * load_elem(v, dtype, voff", "dot += qrow[d] * load_elem(v, dtype, voff"),
    ("rope_sin_sign", "const double ra = a * c - b * sn;", "const double ra = a * c + b * sn;"),
    ("rope_second_of_pair", "const double rb = a * sn + b * c;", "const double rb = b * sn + a * c;"),
    ("rope_pairs_adjacent_halves", "const int ib = layout == 1 ? 2 * i + 1 : i + half;",
     "const int ib = layout == 1 ? 2 * i + 1 : i + 1;"),
    ("rope_offset_dropped", "const int pos = (int)(hs % S) + pos_offset;", "const int pos = (int)(hs % S);"),
    ("rope_frequency_shift", "const double c = (double)cos_tab[(size_t)pos * half + i];",
     "const double c = (double)cos_tab[(size_t)pos * half + (i + 1) % half];"),
    ("rope_sin_from_cos_table", "const double sn = (double)sin_tab[", "const double sn = (double)cos_tab["),
    ("round_ties_away", "(frac == 0.5 && fmod(r, 2.0) != 0.0)", "(frac == 0.5)"),
    ("round_truncates", "if (frac > 0.5 ||", "if (frac > 1.5 ||"),
    ("round_subnormal_spacing", "if (ex < emin) ex = emin;", "if (ex < emin) ex = emin - 1;"),
    ("round_bf16_fraction_bits", "round_to_format(v, 7, -126, 127)", "round_to_format(v, 8, -126, 127)"),
    ("fp16_encode_subnormal", "(uint16_t)(a * ldexp(1.0, 24))", "(uint16_t)(a * ldexp(1.0, 23))"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, tmp_path):
    src = open(obuild.SRC).read()
    assert src.count(old) == 1, "mutation pattern %r must occur exactly once" % name
    mutated = tmp_path / ("attn_oracle_%s.c" % name)
    mutated.write_text(src.replace(old, new))
    lib = obuild.build(str(mutated), str(tmp_path / ("lib_%s.so" % name)))
    orc = oracle.OracleLib(lib)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
        except (ValueError, FloatingPointError, OverflowError):
            failed.append(pin.__name__)
    assert failed, "no pin caught the planted mistake %r" % name
