"""The oracle's pins must catch plausible mistakes.

Each case copies oracle/smla_oracle.c, plants one mistake by text substitution,
builds the copy with gcc in a temporary folder, and runs the pin suite against
it in a subprocess. The suite has to fail for every mutant. Mistakes are only
ever planted in a CPU copy of the oracle.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "smla_oracle.c")

MUTANTS = {
    "scale_group_64": ("scale[i / 128]", "scale[i / 64]"),
    "scale_offset": ("memcpy(scale, row + 512, sizeof scale);", "memcpy(scale, row + 508, sizeof scale);"),
    "rope_offset": ("row + 528 + 2 * r", "row + 526 + 2 * r"),
    "e4m3_bias": ("ldexp(1.0 + (double)m / 8.0, e - 7)", "ldexp(1.0 + (double)m / 8.0, e - 8)"),
    "e4m3_subnormal": ("ldexp((double)m, -9)", "ldexp((double)m, -10)"),
    "drop_rope_in_logits": ("for (int d = 0; d < ORACLE_DQK; ++d)\n                    dot +=",
                            "for (int d = 0; d < ORACLE_DV; ++d)\n                    dot +="),
    "no_softmax_scale": ("s[j] = sm_scale * dot;", "s[j] = dot;"),
    "value_columns_shifted": ("o[d] += p * rows[j * ORACLE_DQK + d];", "o[d] += p * rows[j * ORACLE_DQK + d + 64];"),
    "lse_log2": ("double lse_th = m + log(l);", "double lse_th = m + log2(l);"),
    "table_width_off_by_one": ("if (blk >= max_blocks_per_req)", "if (blk > max_blocks_per_req)"),
    "in_block_offset": ("return (int32_t)(base * ORACLE_BLOCK + off);", "return (int32_t)(base * ORACLE_BLOCK + off + 1);"),
    "weights_unnormalised": ("double p = exp(s[j] - lse_th);", "double p = exp(s[j] - m);"),
    "encode_ties_to_odd": ("smla_oracle_e4m3fn((uint8_t)c) - a);\n        if (d < best_d || (d == best_d && (c & 1) == 0))",
                           "smla_oracle_e4m3fn((uint8_t)c) - a);\n        if (d < best_d || (d == best_d && (c & 1) == 1))"),
    "encode_drops_sign": ("return (uint8_t)(signbit(x) ? (0x80 | best) : best);", "return (uint8_t)best;"),
    "writer_scale_447": ("amax > 0.0f ? amax / 448.0f : 1.0f", "amax > 0.0f ? amax / 447.0f : 1.0f"),
    "writer_scales_reversed": ("memcpy(row + 512 + 4 * g, &scale, sizeof scale);",
                               "memcpy(row + 512 + 4 * (3 - g), &scale, sizeof scale);"),
    "writer_rope_offset": ("memcpy(row + 528, rope, 64 * sizeof(uint16_t));",
                           "memcpy(row + 526, rope, 64 * sizeof(uint16_t));"),
    "ws_start_ignored": ("return workspace_starts[prefill_req] + idx;", "return idx;"),
    "ws_table_width_unchecked": ("if (prefill_req >= num_prefills || idx < 0 || idx / ORACLE_BLOCK >= max_blocks_per_req)",
                                 "if (prefill_req >= num_prefills || idx < 0)"),
    "bf16_truncates": ("nearbyint(ldexp(x, -q))", "trunc(ldexp(x, -q))"),
    "bf16_ties_away": ("nearbyint(ldexp(x, -q))", "round(ldexp(x, -q))"),
    "bf16_nine_bits": ("int q = e - 8;", "int q = e - 9;"),
    "upconvert_rope_offset": ("memcpy(dst + ORACLE_DV, row + 528, 64 * sizeof(uint16_t));",
                              "memcpy(dst + ORACLE_DV, row + 526, 64 * sizeof(uint16_t));"),
    "upconvert_block_of_32": ("int64_t blk = pos / ORACLE_BLOCK;", "int64_t blk = pos / 32;"),
    "chunks_close_early": ("if (r > 0 && used + seq_lens[r] > max_rows) {", "if (r > 0 && used + seq_lens[r] >= max_rows) {"),
    "e2m1_bias": ("v = ldexp(1.0 + (double)m / 2.0, e - 1);", "v = ldexp(1.0 + (double)m / 2.0, e - 2);"),
    "e2m1_subnormal": ("v = ldexp((double)m, -1);", "v = ldexp((double)m, -2);"),
    "nvfp4_nibbles_swapped": ("(i % 2 == 0) ? (uint8_t)(byte & 0xF) : (uint8_t)(byte >> 4)",
                              "(i % 2 == 1) ? (uint8_t)(byte & 0xF) : (uint8_t)(byte >> 4)"),
    "nvfp4_scale_per_32": ("smla_oracle_e4m3fn(row[256 + i / 16])", "smla_oracle_e4m3fn(row[256 + i / 32])"),
    "nvfp4_rope_offset": ("out[ORACLE_DV + r] = smla_oracle_e4m3fn(row[288 + r]);",
                          "out[ORACLE_DV + r] = smla_oracle_e4m3fn(row[287 + r]);"),
    "e2m1_encode_ties_to_odd": ("if (d < best_d || (d == best_d && (c & 1) == 0)) {\n            best = c;\n            best_d = d;\n        }\n    }\n    return (uint8_t)(signbit(x) ? (0x8 | best) : best);",
                                "if (d < best_d || (d == best_d && (c & 1) == 1)) {\n            best = c;\n            best_d = d;\n        }\n    }\n    return (uint8_t)(signbit(x) ? (0x8 | best) : best);"),
    "e2m1_encode_drops_sign": ("return (uint8_t)(signbit(x) ? (0x8 | best) : best);", "return (uint8_t)best;"),
    "nvfp4_writer_scale_amax_over_4": ("smla_oracle_e4m3fn_encode(amax / 6.0f)", "smla_oracle_e4m3fn_encode(amax / 4.0f)"),
    "nvfp4_writer_high_nibble_first": ("row[i / 2] = (uint8_t)(row[i / 2] | (code << 4));",
                                       "row[i / 2] = (uint8_t)((row[i / 2] << 4) | code);"),
    "nvfp4_writer_rope_copied_as_zero": ("row[288 + r] = smla_oracle_e4m3fn_encode((float)smla_oracle_bf16(rope[r]));",
                                         "row[288 + r] = 0;"),
    "nvfp4_attention_reads_fp8_rows": ("smla_oracle_decode_nvfp4_row((const uint8_t *)cache + (int64_t)slot[j] * ORACLE_NVFP4_ROW,",
                                       "smla_oracle_decode_nvfp4_row((const uint8_t *)cache + (int64_t)slot[j] * ORACLE_FP8_ROW,"),
    "nvfp4_upconvert_fp8_stride": ("const int64_t row_bytes = cache_format == 1 ? ORACLE_FP8_ROW : ORACLE_NVFP4_ROW;",
                                   "const int64_t row_bytes = ORACLE_FP8_ROW;"),
    "nvfp4_upconvert_drops_rope": ("for (int i = 0; i < ORACLE_DQK; ++i)\n                    dst[i] = smla_oracle_bf16_rne(v[i]);",
                                   "for (int i = 0; i < ORACLE_DV; ++i)\n                    dst[i] = smla_oracle_bf16_rne(v[i]);"),
    "chunk_starts_not_reset": ("            chunk_ends[n++] = (int32_t)r;\n            used = 0;",
                               "            chunk_ends[n++] = (int32_t)r;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique in the oracle"
    mutant_c = tmp_path / "mutant.c"
    mutant_c.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp", str(mutant_c),
                    "-o", str(so), "-lm"], check=True)
    env = dict(os.environ, SMLA_ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"
