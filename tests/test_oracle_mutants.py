"""Planted mistakes in the oracle are caught by its pins (CPU only).

Each case rewrites one spot of ``oracle/oracle.c`` into a plausible bug (a
dropped term, a wrong sign, an off-by-one mask, a wrong group map, a wrong
index), builds that copy with gcc into a temporary directory, swaps it in for
the real oracle and runs the pin tests.  Every planted mistake must make at
least one pin fail; the unmodified source must pass them all.
"""
import os
import shutil
import subprocess

import pytest

import oracle
from tests import test_oracle_dropout as DR
from tests import test_oracle_fp8 as F
from tests import test_oracle_merge as M
from tests import test_oracle_paged_prefill as C
from tests import test_oracle_pins as P
from tests import test_recurrence_cpu as R

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "scale dropped": ("s[j] = scale * acc;", "s[j] = acc;"),
    "exp sign flipped": ("s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);"),
    "no normalisation": ("for (int c = 0; c < d; ++c) o[c] /= z;", "(void)z;"),
    "lse without max": ("*lse = m + log(z);", "*lse = log(z);"),
    "lse log2": ("*lse = m + log(z);", "*lse = m + log2(z);"),
    "causal excludes diagonal": ("int64_t last = causal ? i + (Nk - Nq) :",
                                 "int64_t last = causal ? i + (Nk - Nq) - 1 :"),
    "causal top-left aligned": ("int64_t last = causal ? i + (Nk - Nq) :",
                                "int64_t last = causal ? i :"),
    "interleaved kv groups": ("        int64_t g = h / group;\n        int64_t last",
                              "        int64_t g = h % Hkv;\n        int64_t last"),
    "values reversed": ("o[c] += w * load(v, dtype, voff[j] + c);",
                        "o[c] += w * load(v, dtype, voff[n - 1 - j] + c);"),
    "key row reversed": ("load(k, dtype, koff[j] + c);", "load(k, dtype, koff[j] + (d - 1 - c));"),
    "bf16 widening": ("uint32_t bits = (uint32_t)((const uint16_t *)p)[i] << 16;",
                      "uint32_t bits = (uint32_t)((const uint16_t *)p)[i] << 15;"),
    "varlen causal off by one": ("int64_t n = causal ? i + 1 : len;", "int64_t n = causal ? i : len;"),
    "paged slot index": ("(t % block_size) * ps[2];", "((t + 1) % block_size) * ps[2];"),
    "paged group map": ("int64_t g = h / group, n = seq_lens[b];",
                        "int64_t g = h % Hkv, n = seq_lens[b];"),
    "max not subtracted in weights": ("s[j] = exp(s[j] - m);", "s[j] = exp(s[j]);"),
    "chunked prefill offset sign": ("int64_t n = causal ? i + 1 + (nk - nq) : nk;",
                                    "int64_t n = causal ? i + 1 - (nk - nq) : nk;"),
    "chunked prefill top-left causal": ("int64_t n = causal ? i + 1 + (nk - nq) : nk;",
                                        "int64_t n = causal ? i + 1 : nk;"),
    "chunked prefill slot index": ("koff[j] = phys * ps[0] + g * ps[1] + (j % block_size) * ps[2];",
                                   "koff[j] = phys * ps[0] + g * ps[1] + (j / block_size) * ps[2];"),
    "chunked prefill block index": ("block_table[seq * (int64_t)max_blocks + j / block_size]",
                                    "block_table[seq * (int64_t)max_blocks + j % block_size]"),
    "e4m3 exponent bias": ("v = ldexp(8.0 + m, e - 10);", "v = ldexp(8.0 + m, e - 11);"),
    "e4m3 subnormal scale": ("v = ldexp((double)m, -9);", "v = ldexp((double)m, -10);"),
    "e4m3 implicit bit dropped": ("v = ldexp(8.0 + m, e - 10);", "v = ldexp((double)m, e - 10);"),
    "e4m3 sign ignored": ("dst[i] = sign ? -v : v;", "dst[i] = v;"),
    "philox key not advanced": ("k0 += W0;", "(void)W0;"),
    "philox products swapped": ("c0 = hi1 ^ c1 ^ k0;", "c0 = hi0 ^ c1 ^ k0;"),
    "philox multipliers swapped": ("p0 = (uint64_t)M0 * c0, p1 = (uint64_t)M1 * c2;",
                                   "p0 = (uint64_t)M1 * c0, p1 = (uint64_t)M0 * c2;"),
    "dropout big-endian byte": ("(out[(j % 16) / 4] >> (8 * (j % 4)))",
                                "(out[(j % 16) / 4] >> (8 * (3 - j % 4)))"),
    "dropout strict threshold": ("return (int)byte >= dp->threshold;", "return (int)byte > dp->threshold;"),
    "dropout scale missing": ("dp ? 256.0 / (256 - dp->threshold) : 1.0", "1.0"),
    "dropout counter word": ("{(uint32_t)(j / 16), (uint32_t)dp->row", "{(uint32_t)(j % 16), (uint32_t)dp->row"),
    "dropout offset ignored": ("(uint32_t)((uint64_t)dp->row >> 32),\n                           dp->offset}",
                               "(uint32_t)((uint64_t)dp->row >> 32),\n                           0u}"),
    "dropout dense row layout": ("dp.row = id; /* (b * Hq + h) * Nq + i */", "dp.row = (h * B + b) * Nq + i;"),
    "dropout packed row layout": ("dp.row = id; /* h * T + t */", "dp.row = t * Hq + h;"),
    "merge lse drops max": ("lse[r] = m + log(z);", "lse[r] = log(z);"),
    "merge unnormalised": ("for (int64_t c = 0; c < d; ++c) orow[c] /= z;", "(void)z;"),
    "merge first part skipped": ("for (int64_t p = 0; p < P; ++p) {\n      const double lp",
                                 "for (int64_t p = 1; p < P; ++p) {\n      const double lp"),
    "merge weight sign": ("const double w = exp(lp - m);", "const double w = exp(m - lp);"),
    "merge parts transposed": ("o_parts[(p * R + r) * d + c]", "o_parts[(r * P + p) * d + c]"),
}

PINS = [
    (P.test_worked_example_merge_rule, {}),
    (P.test_rows_normalised, {"causal": True}),
    (P.test_zero_query_is_mean, {"causal": True}),
    (P.test_single_key, {}),
    (P.test_causal_direction, {}),
    (P.test_causal_prefix_property, {}),
    (P.test_causal_end_aligned_when_more_keys, {}),
    (P.test_gqa_group_mapping, {}),
    (P.test_key_permutation_invariance, {}),
    (P.test_score_shift, {}),
    (P.test_brute_force_twin, {"shape": (2, 5, 7, 4, 2, 3), "causal": True}),
    (P.test_torch_sdpa_fp64, {"shape": (2, 64, 64, 4, 2, 32), "causal": True}),
    (P.test_varlen_equals_dense_per_sequence, {}),
    (P.test_decode_equals_dense_over_gathered_keys, {}),
    (P.test_bf16_widened_exactly, {}),
    (R.test_tiled_causal_equals_oracle, {}),
    (R.test_paged_equals_oracle, {"seq_len": 95}),
    (C.test_chunks_equal_dense_over_gathered_keys, {}),
    (C.test_chunk_longer_than_context_starts_without_keys, {}),
    (F.test_decode_all_codes_match_torch, {}),
    (F.test_decode_closed_forms, {}),
    (DR.test_philox_known_answers, {}),
    (DR.test_keep_decisions_follow_the_counter_layout, {"p": 0.1}),
    (DR.test_zero_probability_is_plain_and_lse_ignores_dropout, {}),
    (DR.test_keep_rate_and_unbiased_scaling, {}),
    (DR.test_single_packed_sequence_numbers_rows_like_dense, {}),
    (DR.test_packed_keep_decisions_use_head_major_rows_and_local_keys, {}),
    (M.test_key_partition_reaches_full_attention, {}),
    (M.test_causal_ring_chunks_merge_to_causal_attention, {}),
    (M.test_worked_example_as_two_parts, {}),
    (M.test_matches_pairwise_recurrence_merge, {}),
    (M.test_special_cases, {}),
]


def _build(tmp_path, text, name):
    src = tmp_path / f"{name}.c"
    src.write_text(text)
    out = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-shared", "-fPIC", str(src), "-o", str(out), "-lm"],
                   check=True, capture_output=True)
    return oracle.load_library(str(out))


def _failures(monkeypatch, lib):
    monkeypatch.setattr(oracle, "_lib", lib)
    failed = []
    for fn, kw in PINS:
        try:
            fn(**kw)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(fn.__name__)
    return failed


@pytest.fixture(scope="module")
def source():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    return open(SRC).read()


def test_unmodified_oracle_passes_all_pins(tmp_path, monkeypatch, source):
    lib = _build(tmp_path, source, "clean")
    assert _failures(monkeypatch, lib) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, monkeypatch, source, name):
    old, new = MUTANTS[name]
    assert source.count(old) >= 1, f"mutation site for {name!r} not found in oracle.c"
    lib = _build(tmp_path, source.replace(old, new), "m_" + name.replace(" ", "_"))
    failed = _failures(monkeypatch, lib)
    assert failed, f"planted mistake {name!r} passed every pin"
