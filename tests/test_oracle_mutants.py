"""Plausible mistakes planted in copies of the oracle (on the CPU) must each
fail at least one pin: evidence that the pins would catch them in the real one."""
import os

import pytest

import oracle
import pins

SRC = open(os.path.join(os.path.dirname(oracle.__file__), "kvc_oracle.c")).read()

MUTANTS = {
    "scale_dropped": ("p[j] = s * scale;", "p[j] = s;"),
    "mask_one_short": ("long last = (long)L - n_q + r;", "long last = (long)L - n_q + r - 1;"),
    "gqa_modulo_map": ("int g = h / G;", "int g = h % Hkv + 0 * G;"),
    "no_max_shift": ("p[j] = exp(p[j] - m);", "p[j] = exp(p[j]);"),
    "no_normalisation": ("= acc / l;", "= acc;"),
    "values_read_from_keys": ("acc += p[j] * load_elem(v, ((size_t)g * L + j) * D + d, dtype);",
                              "acc += p[j] * load_elem(k, ((size_t)g * L + j) * D + d, dtype);"),
    "block_count_floor": ("long have = (len + bs - 1) / bs;", "long have = len / bs;"),
    "free_list_from_back": ("table[(long)b * max_blocks + i] = free_list[*head];",
                            "table[(long)b * max_blocks + i] = free_list[N - 1 - *head];"),
    "append_shifted": ("(size_t)(len + t)) * row;", "(size_t)((len + t + 1) % S_max)) * row;"),
    "slot_offset_shifted": ("(int32_t)(blk * bs + pos % bs);", "(int32_t)(blk * bs + (pos + 1) % bs);"),
    "bf16_ties_away": ("nearbyint(ax / ulp)", "round(ax / ulp)"),
    "combine_unweighted_sum": ("den += exp(cm[c] - M) * cl[c];", "den += cl[c];"),
    "fork_without_reference": ("if (blk >= 0 && blk < N) refs[blk] += 1;",
                               "if (blk >= 0 && blk < N) refs[blk] += 0;"),
    "truncate_keeps_entries": ("      table[(long)b * max_blocks + j] = -1;\n      if (blk < 0 || blk >= N) continue;",
                               "      if (blk < 0 || blk >= N) continue;"),
    "cow_keeps_reference": ("refs[cow_src[b]] -= 1;", "refs[cow_src[b]] -= 0;"),
    "cow_writes_shared_block": ("table[(long)b * max_blocks + len / bs] = cow_dst[b];",
                                "table[(long)b * max_blocks + len / bs] = cow_src[b];"),
    "freed_twice": ("if (i > 0 && cand[i] == cand[i - 1]) continue;", "if (0) continue;"),
    "fp8_bias_off_by_one": ("return fmt == REF_E4M3 ? 7 : 15;", "return fmt == REF_E4M3 ? 8 : 16;"),
    "fp8_ties_up": ("((lo & 1) == 0 ? lo : hi)", "hi"),
    "fp8_scale_not_applied": ("* (double)scales[r];", "* 1.0;"),
    "fp8_amax_of_first_element": ("if (v > amax) amax = v;", "if (d == 0) amax = v;"),
    "mla_scores_from_latent_only": ("        for (int d = 0; d < Dk; ++d)\n          s += load_elem(q, ((size_t)r * Hq + h) * Dk + d, REF_BF16) *",
                                    "        for (int d = 0; d < Dv; ++d)\n          s += load_elem(q, ((size_t)r * Hq + h) * Dk + d, REF_BF16) *"),
    "mla_values_from_row_end": ("acc += p[t] * load_elem(c, (size_t)t * Dk + d, REF_BF16);",
                                "acc += p[t] * load_elem(c, (size_t)t * Dk + d + (Dk - Dv), REF_BF16);"),
    "paged_row_shifted": ("return ((blk * Hkv + g) * bs + j % bs) * D;",
                          "return ((blk * Hkv + g) * bs + (j + 1) % bs) * D;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    assert old in SRC, "mutation site vanished: " + name
    src = tmp_path / "mutant.c"
    src.write_text(SRC.replace(old, new))
    lib = oracle.build(force=True, src=str(src), out=str(tmp_path / "libmutant.so"))
    o = oracle.Oracle(lib)
    failed = []
    for pin in pins.FAST_PINS:
        try:
            pin(o)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, "no pin catches mutant " + name
