"""The oracle's pins must catch plausible mistakes.

Each mutant below is a copy of oracle/swrt_oracle.c with one planted mistake
(an index off by one, a dropped term, a wrong sign, a transposed operand, a
step done in the wrong order, a check weakened). The mutant is compiled with
gcc and the whole pin suite (tests/test_oracle_pins.py, test_oracle_xf_pins.py,
test_oracle_att_pins.py and test_oracle_paged_pins.py) runs against it in its
own process; the suite must fail for every mutant. A mutant that crashes its
process counts as caught. Everything runs on the CPU.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "linear_index_off_by_one": ("j = w + s;", "j = w + s + 1;"),
    "circular_wrong_sign": ("j = floor_mod(floor_mod(w, M) + s, M);",
                            "j = floor_mod(floor_mod(w, M) - s, M);"),
    "modulo_truncates": ("return r < 0 ? r + m : r;", "return r < 0 ? -r : r;"),
    "linear_bound_drops_S": ("(w < 0 || w > M - S)", "(w < 0 || w > M - 1)"),
    "batch_from_last_prefix_dim": ("const int64_t batch_idx = idx[0];",
                                   "const int64_t batch_idx = idx[axis - 1];"),
    "out_of_place_copy_dropped": ("if (present != past && total > 0)",
                                  "if (0 && present != past && total > 0)"),
    "update_rows_reversed": ("(const char *)update + (o * S + s) * row_bytes",
                             "(const char *)update + (o * S + (S - 1 - s)) * row_bytes"),
    "linear_oob_not_flagged": ("set_flag(flags, ORC_FLAG_LINEAR_OOB);", "(void)0;"),
    "total_without_plus_one": ("(int64_t)seqlens_k[b] + 1; /* absolute",
                               "(int64_t)seqlens_k[b]; /* absolute"),
    "total_narrowed_to_32_bits": ("(int64_t)seqlens_k[b] + 1; /* absolute",
                                  "(int64_t)(int32_t)((uint32_t)seqlens_k[b] + 1u); /* absolute"),
    "drift_total_without_plus_one": ("(int64_t)seqlens_k[b] + 1;\n        int64_t P, Lp, L, E;",
                                     "(int64_t)seqlens_k[b];\n        int64_t P, Lp, L, E;"),
    "past_minus_one_not_S": ("P = T - S; /*", "P = T - 1; /*"),
    "past_not_clamped": ("clamped at zero */\n        if (P < 0)\n            P = 0;",
                         "clamped at zero */\n        if (P < -(1LL << 40))\n            P = 0;"),
    "drift_past_not_clamped": ("P = T - S;\n        if (P < 0)\n            P = 0;",
                               "P = T - S;\n        if (P < -(1LL << 40))\n            P = 0;"),
    "resident_off_by_one": ("Lp = P < C ? P : C;", "Lp = P < C ? P : C - 1;"),
    "evict_off_by_one": ("E = Lp + S - C;", "E = Lp + S - C - 1;"),
    "resident_after_drops_E": ("L = Lp + S - E;      /*", "L = Lp + S;      /*"),
    "shift_source_not_offset": ("copy_row(tmp + (r - E) * row_bytes, cache + r * row_bytes,",
                                "copy_row(tmp + (r - E) * row_bytes, cache + (r - E) * row_bytes,"),
    "k_and_v_swapped": ("news[0] = (const char *)k_new;\n    news[1] = (const char *)v_new;",
                        "news[0] = (const char *)v_new;\n    news[1] = (const char *)k_new;"),
    "staged_new_rows_reversed": ("copy_row(stage + (Lp + s) * row_bytes,\n"
                                 "                                     nw + s * nb_stride[2],",
                                 "copy_row(stage + (Lp + s) * row_bytes,\n"
                                 "                                     nw + (S - 1 - s) * nb_stride[2],"),
    "commit_ignores_evictions": ("stage + (E + r) * row_bytes", "stage + r * row_bytes"),
    "new_strides_transposed": ("b * nb_stride[0] + h * nb_stride[1]",
                               "b * nb_stride[1] + h * nb_stride[0]"),
    "staging_slice_stride_C": ("(b * H + h) * (C + S) * row_bytes", "(b * H + h) * C * row_bytes"),
    "length_check_weakened": ("if (Lp < 0 || Lp > C || E < 0 || L > C || L < 1)",
                              "if (Lp < 0 || Lp > C || E < 0)"),
    "drift_gap_too_small": ("const int64_t gap = C - W + 1;", "const int64_t gap = C - W + 2;"),
    "drift_floor_not_ceil": ("(x - C + gap - 1) / gap", "(x - C) / gap"),
    "drift_end_off_by_one": ("L = drift_end(P + S, C, gap);", "L = drift_end(P + S, C, gap) - 1;"),
    "drift_past_from_total": ("Lp = drift_end(P, C, gap);", "Lp = drift_end(P + S, C, gap);"),
    # the fused append's row transform
    "xf_k_and_v_swapped": ("{(const char *)k_new, (const char *)v_new}; /* K, V */",
                           "{(const char *)v_new, (const char *)k_new}; /* K, V */"),
    "xf_lengths_checked_after_positions": ("if (L < 1 || L > C || E < 0 || Lp < 0 || Lp > C)",
                                           "if (0)"),
    "rope_first_sign": ("v[i0] = x0c - x1s;", "v[i0] = x0c + x1s;"),
    "rope_second_sign": ("v[i1] = x1c + x0s;", "v[i1] = x1c - x0s;"),
    "rope_wrong_partner": ("x->interleaved ? 2 * j + 1 : j + half;",
                           "x->interleaved ? 2 * j + 1 : half - 1 - j;"),
    "rope_interleaved_as_half_split": ("const int64_t i0 = x->interleaved ? 2 * j : j;",
                                       "const int64_t i0 = j;"),
    "rope_next_table_row": ("const float *c = x->cos_table + pos * half;",
                            "const float *c = x->cos_table + (pos + 1) * half;"),
    "rope_sin_column_swapped": ("const float *s = x->sin_table + pos * half;",
                                "const float *s = x->cos_table + pos * half;"),
    "rope_rotates_v": ("if (t == 0 && x->cos_table) {\n        /* [GQA-ROPE]",
                       "if (x->cos_table) {\n        /* [GQA-ROPE]"),
    "rope_tail_rotated": ("const int64_t half = x->rotary_dim / 2;",
                          "const int64_t half = head_dim / 2;"),
    "rope_position_cache_relative": ("status = orc_xf_row(x, t, h, past_lens[b] + s,",
                                     "status = orc_xf_row(x, t, h, cache_past_lens[b] + s,"),
    "rope_position_ignores_s": ("status = orc_xf_row(x, t, h, past_lens[b] + s,",
                                "status = orc_xf_row(x, t, h, past_lens[b],"),
    "scatter_position_wrapped": ("status = orc_xf_row(x, t, rank == 4 ? o : 0, w + s,",
                                 "status = orc_xf_row(x, t, rank == 4 ? o : 0, floor_mod(w + s, M),"),
    "rope_range_off_by_one": ("(p0 >= 0 && p0 <= x->max_position - n)",
                              "(p0 >= 0 && p0 <= x->max_position - n + 1)"),
    "rope_range_not_flagged": ("set_flag(flags, ORC_FLAG_ROPE_RANGE);\n            continue;",
                               "continue;"),
    "quant_round_half_up": ("q = nearbyintf(r) + (float)zero_point;",
                            "q = floorf(r + 0.5f) + (float)zero_point;"),
    "quant_zero_point_subtracted": ("q = nearbyintf(r) + (float)zero_point;",
                                    "q = nearbyintf(r) - (float)zero_point;"),
    "quant_truncates": ("q = nearbyintf(r) + (float)zero_point;",
                        "q = truncf(r) + (float)zero_point;"),
    "quant_high_code_wraps": ("        *hi = 127;", "        *hi = 128;"),
    "quant_nan_to_low_code": ("if (isnan(r))\n        return zero_point < lo",
                              "if (isnan(r))\n        return lo + 0 * zero_point;\n    if (0)\n        return zero_point < lo"),
    "quant_v_uses_k_parameters": (": x->scale[t];", ": x->scale[0];"),
    "f32_nan_payload_kept": ("if (isnan(y)) {\n            const uint32_t canonical",
                             "if (0) {\n            const uint32_t canonical"),
    "bf16_ties_away": ("if (dropped > 0x8000 || (dropped == 0x8000 && (kept & 1)))",
                       "if (dropped >= 0x8000)"),
    "bf16_truncates": ("if (dropped > 0x8000 || (dropped == 0x8000 && (kept & 1)))", "if (0)"),
    "f16_rounding_carry_lost": ("if (q == 2048.0) {", "if (q > 2048.0) {"),
    "f16_subnormal_unit": ("const double q = nearbyint(ldexp(a, 24));",
                           "const double q = nearbyint(ldexp(a, 23));"),
    "f16_exponent_bias": ("return sign | (uint16_t)((ex + 15) << 10)",
                          "return sign | (uint16_t)((ex + 14) << 10)"),
    "f16_decode_subnormal": ("v = ldexp((double)m, -24);", "v = ldexp((double)m, -25);"),
    # windowed decode attention
    "att_gqa_modulo": ("const int64_t g = h / group; /* the KV head", "const int64_t g = h % Hkv; /* the KV head"),
    "att_window_one_short": ("const int64_t r0 = L > window ? L - window : 0;",
                             "const int64_t r0 = L > window ? L - window + 1 : 0;"),
    "att_window_one_long": ("const int64_t r0 = L > window ? L - window : 0;",
                            "const int64_t r0 = L > window ? L - window - 1 : 0;"),
    "att_scale_dropped": ("s[r] = scale * dot;", "s[r] = dot;"),
    "att_no_max_shift": ("const double p = exp(s[r] - m);", "const double p = exp(s[r]);"),
    "att_last_row_dropped": ("for (int64_t r = r0; r < L; ++r) { /* softmax", "for (int64_t r = r0; r < L - 1; ++r) { /* softmax"),
    "att_v_from_k": ("const char *vbase = (const char *)v_cache", "const char *vbase = (const char *)k_cache"),
    "att_query_of_kv_head": ("(const char *)q + (b * Hq + h) * D * es", "(const char *)q + (b * Hq + g) * D * es"),
    "att_not_normalised": ("L > r0 ? acc[d] / denom : 0.0", "L > r0 ? acc[d] : 0.0"),
    "bf16_decode_shift": ("uint32_t u = (uint32_t)h << 16;", "uint32_t u = (uint32_t)h << 15;"),
    # paged caches
    "paged_window_one_short": ("T - 1 - left_window > 0 ? T - 1 - left_window : 0",
                               "T - left_window > 0 ? T - left_window : 0"),
    "paged_zero_point_kept": ("return (double)(pg_get_code(fmt, base, i) - zero_point) * (double)scale;",
                              "return (double)pg_get_code(fmt, base, i) * (double)scale;"),
    "paged_codes_high_bits_first": ("const unsigned raw = (byte >> (bit % 8))",
                                    "const unsigned raw = (byte >> ((8 - bits - bit % 8) & 7))"),
    "paged_codes_unsigned": ("if (is_signed && (raw >> (bits - 1)))", "if (0 && is_signed)"),
    "paged_unused_rows_read": ("const float y = r < p->length ? pg_value32(sfmt, ss, sz, src, r * D + e) : 0.0f;",
                               "const float y = pg_value32(sfmt, ss, sz, src, r * D + e);"),
    "paged_contiguity_unchecked": ("} else if (p->start + p->length != end) {", "} else if (0) {"),
    "paged_reads_before_window": ("if (p->start <= r0)\n                        break;",
                                  "if (p->start <= r0)\n                        (void)0;"),
    "paged_append_overwrites": ("pg_store(fmt, sc, zp, base, p->length * D + e,",
                                "pg_store(fmt, sc, zp, base, (p->length - 1) * D + e,"),
    "paged_append_length_kept": ("        p->length += 1;\n", "        (void)0;\n"),
    "paged_dense_target_keeps_parameters": ("/* a dense target has no parameters */\n            sc[t] = 1.0f;\n            zp[t] = 0;\n",
                                            "/* a dense target has no parameters */\n"),
    "paged_live_payload_overwritable": ("return ORC_E_INVALID_ARG; /* the free region holds no live payload */",
                                        "(void)0;"),
    "paged_duplicates_accepted": ("(i > 0 && id <= blocks[i - 1])", "(i > 0 && id < blocks[i - 1])"),
    "paged_destinations_overlap": ("if (dst < next || bytes > free_end - dst)",
                                   "if (bytes > free_end - dst)"),
    # the work prefix of the lengths call
    "work_rows_product_form": ("return (E > 0 ? Lp - E : 0) + 1;", "return E * (Lp - E) + 1;"),
    "work_rows_staged_without_S": ("    return Lp + S;\n}", "    return Lp;\n}"),
    "work_not_a_prefix": ("work_offsets[b + 1] = work_offsets[b] + work_rows(",
                          "work_offsets[b + 1] = work_rows("),
    "work_drift_not_written": ("    work_prefix(cache_past_lens, evict_counts, batch, S, work_offsets);\n    return ORC_OK;\n}\n\n/* ------------------------------------------------------------------------ */\n/* [GQA] windowed step",
                               "    return ORC_OK;\n}\n\n/* ------------------------------------------------------------------------ */\n/* [GQA] windowed step"),
    # per-channel parameters and the fp8 target of the fused append
    "xf_channel_head_ignored": ("x->channel_scale[t][head * head_dim + i]", "x->channel_scale[t][i]"),
    "xf_channel_zero_ignored": ("x->channel_zero_point[t] ? x->channel_zero_point[t][head * head_dim + i]",
                                "0 ? x->channel_zero_point[t][head * head_dim + i]"),
    "fp8_not_scaled": ("c = float_to_e4m3_bits(y / sc);", "c = float_to_e4m3_bits(y);"),
    "fp8_nan_beyond_range": ("return sign | 0x7E; /* +-448; beyond it saturates */",
                             "return a > 448.0 ? 0x7F : (sign | 0x7E);"),
    "fp8_subnormal_truncates": ("q = nearbyint(ldexp(a, 9));", "q = floor(ldexp(a, 9));"),
    "fp8_ties_away": ("q = nearbyint(ldexp(a, 3 - (e - 1)));", "q = round(ldexp(a, 3 - (e - 1)));"),
    "fp8_exponent_bias": ("((e - 1 + 7) << 3)", "((e - 1 + 8) << 3)"),
    "scatter_channel_head_zero": ("status = orc_xf_row(x, t, rank == 4 ? o : 0,",
                                  "status = orc_xf_row(x, t, 0,"),
    "window_channel_head_zero": ("status = orc_xf_row(x, t, h,", "status = orc_xf_row(x, t, 0,"),
    # the sealed-block append and the slotted block table
    "sealed_start_off_by_one": ("T = pages[last].start + pages[last].length;",
                                "T = pages[last].start + pages[last].length - 1;"),
    "sealed_v_over_k": ("dst[1] = dst[0] + bytes[0];", "dst[1] = dst[0];"),
    "sealed_count_kept": ("page_count[s] += 1;", "(void)0;"),
    "sealed_slot_overwrites_last": ("page_ids[p1] = (int32_t)id;",
                                    "page_ids[p1 > p0 ? p1 - 1 : p1] = (int32_t)id;"),
    "sealed_rows_byte_aligned": ("pg_store(fmt[t], sc[t], zp[t], dst[t], r * dim[t] + e,",
                                 "pg_store(fmt[t], sc[t], zp[t], dst[t] + r * ((dim[t] * pg_bits(fmt[t]) + 7) / 8), e,"),
    "sealed_handed_out_id_accepted": ("(last >= first_id && last < first_id + n_streams) ||", ""),
    "sealed_full_not_flagged": ("if (p1 == p0 + page_stride) {", "if (0) {"),
    "sealed_payloads_overlap": ("stride = bytes[0] + bytes[1];", "stride = bytes[0];"),
    "sealed_dense_block_keeps_parameters": ("/* a dense block has no parameters */\n            sc[t] = 1.0f;\n            zp[t] = 0;\n",
                                            "/* a dense block has no parameters */\n"),
    "slotted_range_short": ("*p1 = *p0 + n;", "*p1 = *p0 + n - 1;"),
    "paged_heads_interleaved": ("const int64_t h = g * group + j;", "const int64_t h = j * Hkv + g;"),
    "paged_scale_dropped": ("sc = scale * dot;", "sc = dot;"),
}

# write before shift (the opposite of the order the step formulas list)
_SHIFT_THEN_WRITE = """                    for (int64_t r = E; r < Lp; ++r)
                        copy_row(tmp + (r - E) * row_bytes, cache + r * row_bytes,
                                 row_bytes);
                    for (int64_t r = 0; r < Lp - E; ++r)
                        copy_row(cache + r * row_bytes, tmp + r * row_bytes,
                                 row_bytes);
                    /* write: new tokens -> cache[Lp-E .. Lp-E+S) */
                    for (int64_t s = 0; s < S; ++s)
                        copy_row(cache + (Lp - E + s) * row_bytes,
                                 nw + s * nb_stride[2], row_bytes);
"""
_WRITE_THEN_SHIFT = """                    for (int64_t s = 0; s < S; ++s)
                        copy_row(cache + (Lp - E + s) * row_bytes,
                                 nw + s * nb_stride[2], row_bytes);
                    for (int64_t r = E; r < Lp; ++r)
                        copy_row(tmp + (r - E) * row_bytes, cache + r * row_bytes,
                                 row_bytes);
                    for (int64_t r = 0; r < Lp - E; ++r)
                        copy_row(cache + r * row_bytes, tmp + r * row_bytes,
                                 row_bytes);
"""
MUTANTS["write_before_shift"] = (_SHIFT_THEN_WRITE, _WRITE_THEN_SHIFT)


def _run_pins(lib: str) -> subprocess.CompletedProcess:
    env = dict(os.environ, SWRT_ORACLE_LIB=lib, PYTHONDONTWRITEBYTECODE="1")
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                           os.path.join(ROOT, "tests", "test_oracle_xf_pins.py"),
                           os.path.join(ROOT, "tests", "test_oracle_att_pins.py"),
                           os.path.join(ROOT, "tests", "test_oracle_paged_pins.py")],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


def test_every_mutant_fails_the_pins(tmp_path):
    src = open(oracle.SOURCE).read()
    builds = {}
    for name, (old, new) in MUTANTS.items():
        assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
        path = tmp_path / f"{name}.c"
        path.write_text(src.replace(old, new))
        lib = str(tmp_path / f"lib_{name}.so")
        subprocess.run(["gcc", "-O1", "-std=c11", "-ffp-contract=off", "-shared", "-fPIC",
                        f"-I{os.path.dirname(oracle.SOURCE)}", str(path), "-o", lib, "-lm"],
                       check=True, capture_output=True)
        builds[name] = lib
    with ThreadPoolExecutor(max_workers=max(2, min(8, os.cpu_count() or 2))) as ex:
        results = dict(zip(builds, ex.map(_run_pins, builds.values())))
    survivors = [n for n, r in results.items() if r.returncode == 0]
    assert not survivors, f"mutants not caught by the pins: {survivors}"


def test_unmutated_oracle_passes_the_pins(tmp_path):
    lib = str(tmp_path / "lib_clean.so")
    oracle.build(out=lib)
    r = _run_pins(lib)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
