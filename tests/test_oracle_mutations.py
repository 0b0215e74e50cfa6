"""The pins catch plausible mistakes: each case plants one mistake in a copy
of the oracle source (on the CPU, in a temporary directory), builds it, and
requires the pin suite to fail against that copy.  The committed oracle is
never modified."""
import os
import subprocess
import sys

import pytest

from oracle import build as obuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["tests/test_oracle_quant.py", "tests/test_oracle_transforms.py",
        "tests/test_oracle_layout.py", "tests/test_oracle_scorer.py",
        "tests/test_oracle_sglang.py", "tests/test_oracle_fp8.py", "tests/test_oracle_compressed.py"]

MUTATIONS = {
    "tie_at_0.75_goes_down": ("else if (m < 0.75f) code = 1;", "else if (m <= 0.75f) code = 1;"),
    "tie_at_5_goes_down": ("else if (m <= 5.0f) code = 6;", "else if (m < 5.0f) code = 6;"),
    "zero_code_drops_sign": ("return (uint8_t)((sign << 3) | code);",
                             "return (uint8_t)(((code ? sign : 0) << 3) | code);"),
    "exponent_clamped_at_253": ("    if (e < 1) e = 1;\n    if (e > 254) e = 254;\n    return e;",
                                "    if (e < 1) e = 1;\n    if (e > 253) e = 253;\n    return e;"),
    "floor_exponent_rule": ("uint32_t b = f2u(q);\n    int e = (int)(b >> 23) + ((b & 0x7FFFFFu) != 0u ? 1 : 0);",
                            "uint32_t b = f2u(q);\n    int e = (int)(b >> 23);"),
    "neox_interleaved_swapped": ("int ia = is_neox ? i : 2 * i;", "int ia = is_neox ? 2 * i : i;"),
    "rope_sign": ("S[ia] = round_bf16(ac - bs);", "S[ia] = round_bf16(ac + bs);"),
    "cos_sin_swapped": ("float c = cs_row[i], s = cs_row[ROPE_DIM / 2 + i];",
                        "float s = cs_row[i], c = cs_row[ROPE_DIM / 2 + i];"),
    "no_bf16_after_rope": ("S[ib] = round_bf16(bc + as);", "S[ib] = (bc + as);"),
    "linear_key_scales": ("kv_cache_scale[((blk * 1 + 0) * NGROUPS + g) * BS + (p % 16) * (BS / 16) + p / 16] = e[g];",
                          "kv_cache_scale[((blk * 1 + 0) * NGROUPS + g) * BS + p] = e[g];"),
    "nibbles_swapped": ("bytes[g * (GROUP / 2) + b] = (uint8_t)(lo | (hi << 4));",
                        "bytes[g * (GROUP / 2) + b] = (uint8_t)(hi | (lo << 4));"),
    "q_scales_transposed": ("qs[(g * 16 + h % 16) * J + h / 16] = e[g];",
                            "qs[(g * 16 + h / 16) * J + h % 16] = e[g];"),
    "fwht_sign": ("x[j + h] = u - w;", "x[j + h] = w - u;"),
    "rmsnorm_without_eps": ("float den = sqrtf(mean + eps);", "float den = sqrtf(mean);"),
    "rmsnorm_mean_over_64": ("float mean = p[0] / (float)HEAD_DIM;", "float mean = p[0] / 64.0f;"),
    "bf16_truncates": ("u += 0x7FFFu + lsb;", "u += 0u * lsb;"),
    "bf16_ties_away": ("u += 0x7FFFu + lsb;", "u += 0x8000u + 0u * lsb;"),
    "wrong_rope_slice": ("rope_slice(x + rope_offset, cs_row, is_neox);\n    if (apply_hadamard)",
                         "rope_slice(x + 64 - rope_offset, cs_row, is_neox);\n    if (apply_hadamard)"),
    "q_scale_pads_unwritten": ("memset(qs, 0, (size_t)NGROUPS * 16 * J);", ";"),
    "signed_amax": ("    for (int i = 0; i < n; ++i) {\n        float a = fabsf(v[i]);",
                    "    for (int i = 0; i < n; ++i) {\n        float a = v[i];"),
    "amax_over_4": ("\n    float q = amax / 6.0f;", "\n    float q = amax / 4.0f;"),
    "e4m3_16_signed_amax": ("for (int i = 0; i < 16; ++i) {\n            float a = fabsf(v[i]);",
                            "for (int i = 0; i < 16; ++i) {\n            float a = v[i];"),
    "position_clamp_to_0": ("if (p >= max_pos) p = max_pos - 1;", "if (p >= max_pos) p = 0;"),
    "slot_0_skipped": ("\n        int64_t slot = slot_mapping[t];\n        if (slot < 0 || slot >= nslots) continue;",
                       "\n        int64_t slot = slot_mapping[t];\n        if (slot <= 0 || slot >= nslots) continue;"),
    "fp8_slot_0_skipped": ("const int64_t slot = slot_mapping[t];\n        if (slot < 0 || slot >= nslots) continue;",
                           "const int64_t slot = slot_mapping[t];\n        if (slot <= 0 || slot >= nslots) continue;"),
    "hadamard_scale_1_over_8": ("return (float)(1.0 / sqrt((double)HEAD_DIM));",
                                "return (float)(1.0 / sqrt((double)64));"),
    "weights_head_0_skipped": ("for (int h = 0; h < H; ++h) weights_out[t * H + h] = weights[t * H + h];",
                               "for (int h = 1; h < H; ++h) weights_out[t * H + h] = weights[t * H + h];"),
    "no_saturation": ("else code = 7;", "else code = 6;"),
    "hadamard_scale_before_sums": (
        "    for (int h = 1; h < HEAD_DIM; h <<= 1) {\n        for (int j = 0; j < HEAD_DIM; ++j) {\n            if (j & h) continue;\n            float u = x[j], w = x[j + h];\n            x[j] = u + w;\n            x[j + h] = u - w;\n        }\n    }\n    float sc = hadamard_scale();\n    for (int i = 0; i < HEAD_DIM; ++i) x[i] = round_bf16(x[i] * sc);",
        "    float sc = hadamard_scale();\n    for (int i = 0; i < HEAD_DIM; ++i) x[i] = x[i] * sc;\n    for (int h = 1; h < HEAD_DIM; h <<= 1) {\n        for (int j = 0; j < HEAD_DIM; ++j) {\n            if (j & h) continue;\n            float u = x[j], w = x[j + h];\n            x[j] = u + w;\n            x[j + h] = u - w;\n        }\n    }\n    for (int i = 0; i < HEAD_DIM; ++i) x[i] = round_bf16(x[i]);"),
    "two_stage_sign_on_zero": ("uint8_t sign = (yv < 0.0f && code != 0) ? 1 : 0;",
                               "uint8_t sign = signbit(yv) ? 1 : 0;"),
    "two_stage_reuses_stage_1_exponent": ("int e2 = group_exponent(y, GROUP, floor2);",
                                          "int e2 = e1 + 0 * group_exponent(y, GROUP, floor2);"),
    "two_stage_skips_fake_quant": ("y[i] = e2m1_value(e2m1_nibble(v[i], e1)) * e8m0_value((uint8_t)e1);",
                                   "y[i] = v[i] + 0.0f * e1;"),
    "two_stage_floors_swapped": ("int e1 = group_exponent(v, GROUP, floor1);",
                                 "int e1 = group_exponent(v, GROUP, floor2);"),
    "two_stage_exponents_reversed": ("record[64 + g] = (uint8_t)e2;", "record[64 + 3 - g] = (uint8_t)e2;"),
    "sglang_slot_0_published": ("if (slot <= 0 || slot >= num_slots) continue;",
                                "if (slot < 0 || slot >= num_slots) continue;"),
    "sglang_key_without_norm": ("if (k_norm_gamma) rmsnorm128(x, k_norm_gamma, k_norm_eps);\n        rope_slice(",
                                "if (0) rmsnorm128(x, k_norm_gamma, k_norm_eps);\n        rope_slice("),
    "sglang_query_wrong_rope_slice": ("rope_slice(x + rope_offset, cs_row, is_neox);\n            quantize_row_two_stage",
                                      "rope_slice(x + 64 - rope_offset, cs_row, is_neox);\n            quantize_row_two_stage"),
    "fp8_max_240": ("#define FP8_MAX 448.0f", "#define FP8_MAX 240.0f"),
    "e4m3_ties_up": ("if (r > 0.5 || (r == 0.5 && (si & 1))) si += 1;", "if (r >= 0.5) si += 1;"),
    "e4m3_subnormal_ties_up": ("if (r > 0.5 || (r == 0.5 && (ki & 1))) ki += 1;",
                               "if (r >= 0.5) ki += 1;"),
    "e4m3_zero_sign_dropped": ("const uint8_t sign = signbit(y) ? 0x80 : 0x00;",
                               "const uint8_t sign = (y < 0.0f) ? 0x80 : 0x00;"),
    "fp8_ue8m0_floor_rule": ("uint32_t b = f2u(s);\n        int e = (int)(b >> 23) + ((b & 0x7FFFFFu) != 0u ? 1 : 0);",
                             "uint32_t b = f2u(s);\n        int e = (int)(b >> 23);"),
    "fp8_fold_without_weights_scale": ("f32_to_bf16_bits(w * weights_scale);",
                                       "f32_to_bf16_bits(w + 0.0f * weights_scale);"),
    "fp8_fold_truncates": ("f32_to_bf16_bits(w * weights_scale);",
                           "(uint16_t)(f2u(w * weights_scale) >> 16);"),
    "fp8_multiplies_by_scale": ("codes[i] = e4m3_code(x[i] / s);", "codes[i] = e4m3_code(x[i] * s);"),
    "fp8_key_scale_misplaced": ("kv_cache_scale[slot] = quantize_row_fp8(",
                                "kv_cache_scale[slot ^ 1] = quantize_row_fp8("),
    "fp8_floor_ignored": ("if (s < scale_floor) s = scale_floor;", "if (0) s = scale_floor;"),
    "compress_ratio_ignored": ("pos -= pos % compress_ratio;    /* RoPE at the group's first position */",
                               "pos -= 0 * compress_ratio;"),
    "fake_quant_ratio_ignored": ("pos -= pos % compress_ratio;\n        float v[HEAD_DIM];",
                                 "pos -= 0 * compress_ratio;\n        float v[HEAD_DIM];"),
    "e4m3_16_amax_over_4": ("float q = amax / 6.0f;\n        if (q < scale_floor) q = scale_floor;\n        const float s = e4m3_value",
                            "float q = amax / 4.0f;\n        if (q < scale_floor) q = scale_floor;\n        const float s = e4m3_value"),
    "e4m3_16_scale_not_rounded": ("const float s = e4m3_value(e4m3_code(q));",
                                  "const float s = q + 0.0f * e4m3_value(e4m3_code(q));"),
    "e4m3_16_zero_scale_unsigned": ("out = copysignf(0.0f, v[i]);", "out = 0.0f;"),
    "fake_quant_ue8m0_unscaled": ("const float q = e2m1_value(e2m1_nibble(v[i], e)) * e8m0_value((uint8_t)e);",
                                  "const float q = e2m1_value(e2m1_nibble(v[i], e));"),
    "sglang_query_heads_shifted": ("q_packed + (t * H + h) * SLOT68", "q_packed + (t * H + (h ^ 1)) * SLOT68"),
}


# Scorer mistakes, each of which the hand-derived worked cases alone must catch
# (tests/golden/scorer_worked_cases.json: values derived by hand, not by
# re-evaluating the oracle's formula).
SCORER_PINS = ["tests/test_oracle_scorer.py::test_scorer_worked_cases"]
SCORER_MUTATIONS = {
    "scorer_without_relu": ("double score = (apply_relu && dot < 0.0) ? 0.0 : dot;",
                            "double score = dot;"),
    "scorer_mask_off_by_one": ("if (s > pos || blk < 0 || blk >= NB) {",
                               "if (s >= pos || blk < 0 || blk >= NB) {"),
    "scorer_invalid_block_read": ("if (s > pos || blk < 0 || blk >= NB) {",
                                  "if (s > pos || blk >= NB) { if (blk < 0) blk = 0;"),
    "scorer_ignores_weights": ("acc += w * score;", "acc += score;"),
    "scorer_relu_after_weighting": ("acc += w * score;",
                                    "acc += (apply_relu && w * dot < 0.0) ? 0.0 : w * dot;"),
    "scorer_ignores_weights_scale": ("*out = (float)((double)weights_scale * acc);",
                                     "*out = (float)(acc + 0.0 * weights_scale);"),
    "scorer_linear_key_scales": ("(p % 16) * (KV_BLOCK / 16) + p / 16];", "p];"),
    "scorer_query_scale_transposed": ("q_scale_out[t * (int64_t)NGROUPS * 16 * J + (g * 16 + h % 16) * J + h / 16];",
                                      "q_scale_out[t * (int64_t)NGROUPS * 16 * J + (g * 16 + h / 16) * J + h % 16];"),
}


def _run_mutant(name, workdir):
    old, new = MUTATIONS[name] if name in MUTATIONS else SCORER_MUTATIONS[name]
    pins = PINS if name in MUTATIONS else SCORER_PINS
    src = open(obuild.SRC).read()
    if src.count(old) != 1:
        return f"mutation site not unique or missing: {name}"
    d = os.path.join(workdir, name)
    os.makedirs(d, exist_ok=True)
    mutant = os.path.join(d, "fp4idx_oracle_mutant.c")
    with open(mutant, "w") as f:
        f.write(src.replace(old, new))
    lib = obuild.build(src=mutant, out=os.path.join(d, "libmutant.so"))
    env = dict(os.environ, FP4IDX_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", *pins], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    return r.returncode


@pytest.fixture(scope="module")
def mutant_results(tmp_path_factory):
    from concurrent.futures import ThreadPoolExecutor

    workdir = str(tmp_path_factory.mktemp("mutants"))
    workers = max(1, min(6, (os.cpu_count() or 2) - 1))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        futs = {n: ex.submit(_run_mutant, n, workdir)
                for n in sorted(MUTATIONS) + sorted(SCORER_MUTATIONS)}
        return {n: f.result() for n, f in futs.items()}


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTATIONS) + sorted(SCORER_MUTATIONS))
def test_pins_catch_planted_mistake(name, mutant_results):
    rc = mutant_results[name]
    assert not isinstance(rc, str), rc
    assert rc != 0, f"no pin caught the planted mistake {name}"
