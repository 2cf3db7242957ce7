"""Plausible mistakes planted in a copy of the oracle (on the CPU) must each
fail at least one pin: evidence that the pins constrain every part of the
oracle (mask predicate, alignment, GQA mapping, scale, normaliser, LSE,
operand choice, layouts, packed and decode indexing)."""
import os

import pytest

import oracle
from oracle_pins import PINS

MUTANTS = {
    "top_left_alignment": ("long pos = i + (sk - sq);", "long pos = i;"),
    "causal_off_by_one": ("if (causal && j > pos) return 0;", "if (causal && j >= pos) return 0;"),
    "window_left_exclusive": ("if (wl >= 0 && j < pos - wl) return 0;",
                              "if (wl >= 0 && j <= pos - wl) return 0;"),
    "window_right_ignored_at_zero": ("if (wr >= 0 && j > pos + wr) return 0;",
                                     "if (wr > 0 && j > pos + wr) return 0;"),
    "window_sides_swapped": ("if (wl >= 0 && j < pos - wl) return 0;",
                             "if (wr >= 0 && j < pos - wr) return 0;"),
    "dropped_scale": ("scores[j] = scale * dot(qrow, k + j * kv_stride, d);",
                      "scores[j] = dot(qrow, k + j * kv_stride, d);"),
    "lse_without_max": ("*lse = m + log(l);", "*lse = log(l);"),
    "unnormalised_weights": ("double p = exp(scores[j] - m) / l;",
                             "double p = exp(scores[j] - m);"),
    "sum_without_max_shift": ("l += exp(scores[j] - m);", "l += exp(scores[j]);"),
    "keys_used_as_values": ("const double* vrow = v + j * kv_stride;",
                            "const double* vrow = k + j * kv_stride;"),
    "gqa_modulo_mapping": ("int g = h / G;\n                        const double* qrow",
                           "int g = h % Hkv;\n                        const double* qrow"),
    "kv_head_ignored": ("                        const double* kb = k + ((long)b * Sk * Hkv + g) * d;",
                        "                        const double* kb = k + ((long)b * Sk * Hkv) * d;"),
    "bwd_kv_head_ignored": ("for (int g = 0; g < Hkv; ++g) {\n                    const double* kb = k + ((long)b * Sk * Hkv + g) * d;",
                            "for (int g = 0; g < Hkv; ++g) {\n                    const double* kb = k + ((long)b * Sk * Hkv) * d;"),
    "q_layout_bhsd": ("const double* qrow = q + (((long)b * Sq + i) * Hq + h) * d;",
                      "const double* qrow = q + (((long)b * Hq + h) * Sq + i) * d;"),
    "lse_layout_bsh": ("double* l = lse + ((long)b * Hq + h) * Sq + i;",
                       "double* l = lse + ((long)b * Sq + i) * Hq + h;"),
    "varlen_global_row_index": ("long i = t - cu_q[z];", "long i = t;"),
    "varlen_key_offset_from_q": ("const double* kb = k + ((long)cu_k[z] * Hkv + g) * d;",
                                 "const double* kb = k + ((long)cu_q[z] * Hkv + g) * d;"),
    "decode_reads_whole_cache": ("long sk = cache_seqlens[b];", "long sk = Sk_cap;"),
    "decode_gqa_modulo": ("int g = h / G;\n                    const double* kb = kc",
                          "int g = h % Hkv;\n                    const double* kb = kc"),
    "max_not_tracked": ("if (scores[j] > m) m = scores[j];", "if (m == -INFINITY) m = scores[j];"),
    "bwd_missing_row_term": ("const double ds = p[j] * (dp[j] - D);", "const double ds = p[j] * dp[j];"),
    "bwd_sign_flipped": ("const double ds = p[j] * (dp[j] - D);", "const double ds = p[j] * (D - dp[j]);"),
    "bwd_dq_without_scale": ("dqrow[c] += scale * ds * krow[c];", "dqrow[c] += ds * krow[c];"),
    "bwd_dk_from_keys": ("dkrow[c] += scale * ds * qrow[c];", "dkrow[c] += scale * ds * krow[c];"),
    "bwd_unnormalised_weights": ("p[j] = exp(p[j] - m) / l;", "p[j] = exp(p[j] - m);"),
    "bwd_dp_from_keys": ("dp[j] = dot(gorow, vb + j * kvs, d);", "dp[j] = dot(gorow, kb + j * kvs, d);"),
    "bwd_first_group_head_only": ("for (int h = g * G; h < (g + 1) * G; ++h)",
                                  "for (int h = g * G; h < g * G + 1; ++h)"),
    "bwd_dv_from_queries": ("dvrow[c] += p[j] * gorow[c];", "dvrow[c] += p[j] * qrow[c];"),
    "paged_gather_ignores_table": (
        "                        long pg = block_table[(long)b * max_pages + t / page_size];",
        "                        long pg = (long)b * max_pages + t / page_size;"),
    "paged_table_row_stride": (
        "                        long pg = block_table[(long)b * max_pages + t / page_size];",
        "                        long pg = block_table[(long)b + t / page_size];"),
    "paged_row_ignores_offset": ("                        long row = pg * page_size + t % page_size;",
                                 "                        long row = pg * page_size;"),
    "append_not_seen": ("long sk = (long)cache_seqlens[b] + append;", "long sk = (long)cache_seqlens[b];"),
    "append_value_from_key": ("v_pages[(row * Hkv + g) * d + c] = v_new[((long)b * Hkv + g) * d + c];",
                              "v_pages[(row * Hkv + g) * d + c] = k_new[((long)b * Hkv + g) * d + c];"),
    "alibi_sign_flipped": ("s -= slope * fabs((double)(pos - j));", "s += slope * fabs((double)(pos - j));"),
    "alibi_without_abs": ("s -= slope * fabs((double)(pos - j));", "s -= slope * (double)(pos - j);"),
    "alibi_kv_head_slope": ("double slope = alibi ? alibi[h] : 0.0;", "double slope = alibi ? alibi[g] : 0.0;"),
    "alibi_top_left": ("long pos = i + sk - sq;", "long pos = i;"),
    "softcap_not_divided": ("if (softcap > 0) s = softcap * tanh(s / softcap);",
                            "if (softcap > 0) s = softcap * tanh(s);"),
    "softcap_ignored": ("if (softcap > 0) s = softcap * tanh(s / softcap);", "if (softcap > 0) s = s;"),
    "append_head_ignored": ("k_pages[(row * Hkv + g) * d + c] = k_new[((long)b * Hkv + g) * d + c];",
                            "k_pages[(row * Hkv + g) * d + c] = k_new[((long)b * Hkv) * d + c];"),
    # the row-sampled entry: the row's own index, and its sequence's query count
    "rows_index_is_sample_position": ("kv_stride, qi[r], sq, sk, d,", "kv_stride, (int64_t)r, sq, sk, d,"),
    "rows_query_count_from_keys": ("kv_stride, qi[r], sq, sk, d,", "kv_stride, qi[r], sk, sk, d,"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.oracle.SRC).read()
    assert src.count(old) == 1, f"mutation site not unique: {name}"
    mut_src = tmp_path / "fa_oracle_mut.c"
    mut_src.write_text(src.replace(old, new))
    lib_path = str(tmp_path / "libfa_oracle_mut.so")
    oracle.build(str(mut_src), lib_path)
    orc = oracle.Oracle(oracle.load(lib_path))
    failed = []
    for pin in PINS:              # the first failing pin is enough
        try:
            pin(orc)
        except (AssertionError, RuntimeError, FloatingPointError, ValueError):
            failed.append(pin.__name__)
            break
    assert failed, f"mutant {name} passed every pin"
