"""Planted mistakes in the oracle must fail at least one pin (CPU only).

Each case copies oracle/oracle.c, applies one textual mutation (a dropped term, a flipped
sign or comparison, a wrong index, a transposed operand, a wrong scale, ...), builds the
mutant with gcc into a temporary directory and runs every pin from oracle_pins against it.
The unmodified oracle passes all pins (test_oracle.py); every mutant must fail one.
"""
import os
import shutil
import subprocess

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, original text, replacement, expected number of occurrences)
MUTANTS = [
    ("gap_sign_flipped", "return tile_max - running_max;", "return running_max - tile_max;", 1),
    ("skip_comparison_flipped", "unit_gap < u->tau", "unit_gap > u->tau", 1),
    ("skip_comparison_not_strict", "unit_gap < u->tau", "unit_gap <= u->tau", 1),
    ("unit_gap_min_over_rows", "if (g > G) G = g;", "if (voters == 1 || g < G) G = g;", 2),
    ("first_tile_gap_not_infinite", "return INFINITY;  /* first tile", "return tile_max;  /* first tile", 1),
    ("causal_off_by_one", "(s->causal ? off + i + 1 : Sk)", "(s->causal ? off + i : Sk)", 1),
    ("gqa_head_map_modulo", "g = h / G,", "g = h % s->Hkv,", 1),
    ("scale_1_over_d", "1.0 / sqrt((double)s->d)", "1.0 / (double)s->d", 2),
    ("values_read_from_keys", "load_row(u, u->v, j, row);", "load_row(u, u->k, j, row);", 2),
    ("normaliser_drops_first_key", "if (m > -INFINITY)\n      for (int j = 0;", "if (m > -INFINITY)\n      for (int j = 1;", 1),
    ("no_rescale_in_scan", "l[r] *= c;", "l[r] *= 1.0;", 1),
    ("running_max_not_reset_per_split",
     "for (int r = 0; r < nr; ++r) R[r] = u->seed_scans && s > 0 && nt > 0 ? M[(int64_t)r * nt] : -INFINITY;",
     "if (s == 0) for (int r = 0; r < nr; ++r) R[r] = -INFINITY;", 1),
    ("sink_seed_from_split_first_tile", "? M[(int64_t)r * nt] :", "? M[(int64_t)r * nt + u->scan_first[s]] :", 1),
    ("sink_seed_from_tile_one", "? M[(int64_t)r * nt] :", "? M[(int64_t)r * nt + (nt > 1)] :", 1),
    ("sink_seed_ignored_in_scan_form", "double run = s > 0 && seed[r] > m[r] ? seed[r] : m[r];", "double run = m[r];", 1),
    ("sink_seed_flag_dropped", "u.seed_scans = s->sink_seed != 0;", "u.seed_scans = 0;", 1),
    ("fp8_exponent_bias_8", "ldexp((double)(8 + m), e - 10)", "ldexp((double)(8 + m), e - 11)", 1),
    ("fp8_subnormals_as_normals", "e == 0 ? ldexp((double)m, -9) :", "e < 0 ? ldexp((double)m, -9) :", 1),
    ("fp8_k_scale_dropped", "u.k_mul = s->k_scale > 0 ? s->k_scale : 1.0;", "u.k_mul = 1.0;", 1),
    ("chunk_top_left_causal", "limit[r] = i < s->S ? (s->causal ? off + i + 1 : Sk) : 0;",
     "limit[r] = i < s->S ? (s->causal ? i + 1 : Sk) : 0;", 1),
    ("chunk_offset_off_by_one", "limit[r] = i < s->S ? (s->causal ? off + i + 1 : Sk) : 0;",
     "limit[r] = i < s->S ? (s->causal ? off + i + 2 : Sk) : 0;", 1),
    ("chunk_tiles_without_offset", "u.ntiles = s->causal ? (off + i1 - 1) / s->tile_k + 1 : P->nkt;",
     "u.ntiles = s->causal ? (i1 - 1) / s->tile_k + 1 : P->nkt;", 1),
    ("fp8_v_scale_on_keys", "const double mul = src == u->k ? u->k_mul : u->v_mul;",
     "const double mul = src == u->k ? u->v_mul : u->v_mul;", 1),
    ("combine_equal_weights", "double w = exp(ls[(int64_t)s * nr + r] - big);", "double w = ls[(int64_t)s * nr + r] > -INFINITY ? 1.0 : 0.0;", 1),
    ("tile_max_includes_next_key", "j < (t + 1) * T && j < nk", "j <= (t + 1) * T && j < nk", 1),
    ("bf16_shift_15", "[i] << 16;", "[i] << 15;", 1),
    ("bf16_low_half_of_word", "uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;",
     "uint32_t bits = (uint32_t)((const uint16_t*)base)[i];", 1),
    ("f32_truncated_to_bf16", "if (dt == ORACLE_F32) return (double)((const float*)base)[i];",
     "if (dt == ORACLE_F32) { uint32_t u; memcpy(&u, (const float*)base + i, 4); u &= 0xffff0000u; float f; "
     "memcpy(&f, &u, 4); return (double)f; }", 1),
    ("dtype_codes_swapped", "if (dt == ORACLE_F32) return", "if (dt == ORACLE_BF16) return", 1),
    ("pot_floor_not_nearest", "return nearbyint(logit * 1.4426950408889634074);",
     "return floor(logit * 1.4426950408889634074);", 1),
    ("pot_natural_log_units", "return nearbyint(logit * 1.4426950408889634074);", "return nearbyint(logit);", 1),
    ("pot_difference_rounded", "ldexp(1.0, (int)(pot_exponent(l) - pot_exponent(mu[r])))",
     "ldexp(1.0, (int)pot_exponent(l - mu[r]))", 1),
    ("pot_ignored_in_scan_form", "double p = u->pot ? ldexp(1.0, (int)(pot_exponent(x) - kref[r])) : exp(x - m[r]);",
     "double p = exp(x - m[r]);", 1),
    ("pot_flag_dropped", "u.pot = s->weights == ORACLE_WEIGHTS_ROWMAX_POT;", "u.pot = 0;", 1),
    ("split_size_floor", "const int tps = (nt + P - 1) / P;", "const int tps = nt / P > 0 ? nt / P : 1;", 1),
]


@pytest.fixture(scope="module")
def workdir(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    return tmp_path_factory.mktemp("mutants")


@pytest.mark.parametrize("name,orig,repl,count", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(workdir, name, orig, repl, count):
    src = open(SRC).read()
    assert src.count(orig) == count, f"mutation site for {name} not found as expected"
    d = workdir / name
    d.mkdir()
    shutil.copy(os.path.join(os.path.dirname(SRC), "oracle.h"), d / "oracle.h")
    (d / "oracle.c").write_text(src.replace(orig, repl))
    so = str(d / "liboracle_mutant.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", str(d / "oracle.c"), "-o", so,
                    "-lpthread", "-lm"], check=True)
    lib = oracle.load(so)
    failed = oracle_pins.run_all(lib)
    assert failed, f"mutant {name} passed every pin"
