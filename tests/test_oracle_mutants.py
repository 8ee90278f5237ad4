"""Planted mistakes in the oracle must be caught by its pins (no GPU).

Each mutant is a copy of ``oracle/ep_oracle.c`` with one plausible mistake
(an off-by-one slot, the wrong expert placement, a dropped rank dedup, the
wrong rounding tie rule, a transposed division, swapped FMA operands, ...),
compiled with gcc into a temporary directory and run through every pin in a
child process.  The test fails if any mutant passes every pin."""
import concurrent.futures
import os
import subprocess
import sys
import tempfile

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))

# (name, [(exact text in ep_oracle.c, replacement), ...])
COMBINE_YR = "const uint16_t *yr = y + ((size_t)e * S + j) * H;\n            float w = topk_weights[i];"
COMBINE_FMA = "\n            for (int32_t c = 0; c < H; ++c)\n                acc[c] = fmaf(w, oracle_bf16_to_f32(yr[c]), acc[c]);"
COMBINE_INIT = ("            acc[c] = 0.0f;\n        for (int32_t k = 0; k < K; ++k) {\n"
                "            size_t i = (size_t)t * K + k;\n"
                "            int32_t e = routed_expert(topk_idx[i], E, &status);\n"
                "            if (e < 0)\n                continue;\n            int32_t j = expert_slot[i];")
PACK_STORE = "size_t row = (size_t)e * S + j;\n            payload_store(&p, xt, row, recv_x, recv_scales);\n"
NORMAL_ROW = "size_t row = (size_t)r * M + j;\n            payload_store(&p, xt, row, recv_x, recv_scales);"
NORMAL_COMBINE_ROW = "size_t row = (size_t)r * M + j;\n            const uint16_t *yr = y + row * H;"

MUTANTS = [
    ("slot_off_by_one", [("expert_slot[i] = num_tokens_per_expert[e];",
                          "expert_slot[i] = num_tokens_per_expert[e] + 1;")]),
    ("interleaved_placement", [("return e / (E / R);", "return e % R;")]),
    ("no_rank_dedup", [("in_set[rank_of(e, E, R)] = 1;", "in_set[rank_of(e, E, R)] += 1;"),
                       ("num_tokens_per_rank[r] += 1;", "num_tokens_per_rank[r] += in_set[r];")]),
    ("inclusive_offsets", [("expert_offset[e] = run;\n            run += num_tokens_per_expert[e];",
                            "run += num_tokens_per_expert[e];\n            expert_offset[e] = run;")]),
    ("masked_as_expert0", [("if (id == -1)\n        return -1;", "if (id == -1)\n        return 0;")]),
    ("rank_slot_not_reset", [("rank_slot[i] = -1;", "rank_slot[i] = 0;")]),
    ("bf16_round_half_up", [("if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))",
                             "if (dropped >= 0x8000u)")]),
    ("bf16_truncate", [("        kept += 1u;", "        kept += 0u;")]),
    ("fp8_ties_away", [("double m = nearbyint((ldexp(a, -e) - 1.0) * 8.0);",
                        "double m = round((ldexp(a, -e) - 1.0) * 8.0);")]),
    ("fp8_bias_8", [("(((e + 7) << 3)", "(((e + 8) << 3)")]),
    ("fp8_subnormal_step", [("nearbyint(a * 0x1p9)", "nearbyint(a * 0x1p10)")]),
    ("fp8_decode_bias", [("ldexp((double)(8 + m), E - 10)", "ldexp((double)(8 + m), E - 11)")]),
    ("inv_transposed", [("float inv = 448.0f / ap;", "float inv = ap / 448.0f;")]),
    ("scale_inverted", [("float scale = ap / 448.0f;", "float scale = 448.0f / ap;")]),
    ("no_amax_floor", [("return (a > 1e-4f) ? a : 1e-4f;", "return (a > 0.0f) ? a : 1.0f;")]),
    ("amax_signed", [("float m = fabsf(oracle_bf16_to_f32(xb[c]));",
                      "float m = oracle_bf16_to_f32(xb[c]);")]),
    ("fma_operands_swapped", [(COMBINE_YR + COMBINE_FMA, COMBINE_YR + COMBINE_FMA.replace(
        "fmaf(w, oracle_bf16_to_f32(yr[c]), acc[c])", "fmaf(w, acc[c], oracle_bf16_to_f32(yr[c]))"))]),
    ("weight_of_first_k", [(COMBINE_YR, COMBINE_YR.replace("topk_weights[i]", "topk_weights[(size_t)t * K]"))]),
    ("combine_acc_negzero", [(COMBINE_INIT, COMBINE_INIT.replace("acc[c] = 0.0f;", "acc[c] = -0.0f;"))]),
    ("src_idx_is_k", [(PACK_STORE + "            recv_src_idx[row] = t;",
                       PACK_STORE + "            recv_src_idx[row] = k;")]),
    ("scales_row_stride", [("memcpy((float *)recv_scales + row * G, p->sc",
                            "memcpy((float *)recv_scales + row, p->sc")]),
    ("dequant_wrong_block", [("float v = qv * scales[c / 128];", "float v = qv * scales[c % (H / 128)];")]),
    ("pow2_steps_past_equality", [("while (ldexp(448.0, e) < (double)ap)", "while (ldexp(448.0, e) <= (double)ap)")]),
    ("pow2_search_starts_high", [("    e -= 9;", "    e -= 7;")]),
    ("ue8m0_bias_128", [("(uint32_t)(p->ex[b] + 127) << (8 * (b % 4))", "(uint32_t)(p->ex[b] + 128) << (8 * (b % 4))")]),
    ("ue8m0_byte_order", [("<< (8 * (b % 4))", "<< (8 * (3 - b % 4))")]),
    # expand layout (Ascend deep dive, phase 1)
    ("aligned_floor", [("run += (counts[e] + a - 1) / a * a;", "run += counts[e] / a * a;")]),
    ("aligned_pads_full_queues", [("run += (counts[e] + a - 1) / a * a;", "run += (counts[e] / a + 1) * a;")]),
    ("expand_padding_not_zeroed", [("payload_zero(&p, (size_t)row, recv_x, recv_scales);", "")]),
    ("expand_padding_src_zero", [("recv_src_idx[row] = -1;", "recv_src_idx[row] = 0;")]),
    ("expand_next_queue", [("int64_t row = (int64_t)expert_offset[e] + expert_slot[i];\n"
                            "            if (expert_slot[i] < 0 || row >= expert_offset[e + 1] || expert_offset[e + 1] > T) {\n"
                            "                status |= ORACLE_BAD_SLOT;\n                continue;\n            }\n"
                            "            payload_store",
                            "int64_t row = (int64_t)expert_offset[e] + expert_slot[i] + 1;\n"
                            "            if (expert_slot[i] < 0 || row > expert_offset[e + 1] || expert_offset[e + 1] > T) {\n"
                            "                status |= ORACLE_BAD_SLOT;\n                continue;\n            }\n"
                            "            payload_store")]),
    # normal mode ([V1] §5.1)
    ("normal_global_ids", [("local ? (int64_t)(e - r * L) : -1;", "local ? (int64_t)e : -1;")]),
    ("normal_weights_not_masked", [("recv_topk_weights[row * K + k] = local ? topk_weights[i] : 0.0f;",
                                    "recv_topk_weights[row * K + k] = topk_weights[i];")]),
    ("normal_row_transposed", [(NORMAL_ROW, NORMAL_ROW.replace("(size_t)r * M + j", "(size_t)j * R + r"))]),
    ("normal_combine_row_transposed", [(NORMAL_COMBINE_ROW,
                                        NORMAL_COMBINE_ROW.replace("(size_t)r * M + j", "(size_t)j * R + r"))]),
    ("normal_combine_overwrites", [("acc[c] = acc[c] + oracle_bf16_to_f32(yr[c]);",
                                    "acc[c] = oracle_bf16_to_f32(yr[c]);")]),
    ("normal_weights_overwrite", [("wacc[k] = wacc[k] + recv_topk_weights[row * K + k];",
                                   "wacc[k] = recv_topk_weights[row * K + k];")]),
    # shared-expert bias (Ascend deep dive, "Combine: More Output, Same Cost")
    ("bias_added_first", [
        (COMBINE_INIT, COMBINE_INIT.replace(
            "acc[c] = 0.0f;", "acc[c] = bias ? oracle_bf16_to_f32(bias[(size_t)t * H + c]) : 0.0f;")),
        (COMBINE_YR + COMBINE_FMA + "\n        }\n        add_bias_row(acc, bias ? bias + (size_t)t * H : NULL, H);",
         COMBINE_YR + COMBINE_FMA + "\n        }")]),
    ("bias_overwrites", [("acc[c] = acc[c] + oracle_bf16_to_f32(bias_row[c]);",
                          "acc[c] = oracle_bf16_to_f32(bias_row[c]);")]),
    # group-limited gating
    ("gating_group_sum", [("                    if (st[g * L + i] > gs[g])\n                        gs[g] = st[g * L + i];",
                           "                    gs[g] = gs[g] + st[g * L + i];")]),
    ("gating_sum_descending", [("for (int32_t i = 0; i < L; ++i)\n                    acc = acc + st[g * L + i];",
                                "for (int32_t i = L - 1; i >= 0; --i)\n                    acc = acc + st[g * L + i];")]),
    ("gating_sum_in_double", [("float acc = 0.0f;\n                for (int32_t i = 0; i < L; ++i)\n                    acc = acc + st[g * L + i];\n                gs[g] = acc;",
                               "double acc = 0.0;\n                for (int32_t i = 0; i < L; ++i)\n                    acc = acc + st[g * L + i];\n                gs[g] = (float)acc;")]),
    ("gating_sum_is_max", [("                    acc = acc + st[g * L + i];",
                            "                    acc = (i == 0 || st[g * L + i] > acc) ? st[g * L + i] : acc;")]),
    ("gating_sum_rule_softmax", [("z[k] = rule == ORACLE_GATE_MAX_SOFTMAX ? exp(v - top) : 1.0 / (1.0 + exp(-v));",
                                  "z[k] = exp(v - top);")]),
    ("gating_sigmoid_sign", [("1.0 / (1.0 + exp(-v))", "1.0 / (1.0 + exp(v))")]),
    ("gating_group_ties_high", [("if (!kept[g] && (best < 0 || gs[g] > gs[best]))",
                                 "if (!kept[g] && (best < 0 || gs[g] >= gs[best]))")]),
    ("gating_expert_ties_high", [("if (kept[e / L] && !taken[e] && (best < 0 || st[e] > st[best]))",
                                  "if (kept[e / L] && !taken[e] && (best < 0 || st[e] >= st[best]))")]),
    ("gating_ignores_groups", [("if (kept[e / L] && !taken[e] && (best < 0 || st[e] > st[best]))",
                                "if (!taken[e] && (best < 0 || st[e] > st[best]))")]),
    ("gating_group_of_expert", [("if (kept[e / L] && !taken[e]", "if (kept[e % G] && !taken[e]")]),
    ("gating_one_group_short", [("for (int32_t n = 0; n < TG; ++n) {", "for (int32_t n = 1; n < TG; ++n) {")]),
    ("gating_unnormalised", [("topk_weights[(size_t)t * K + k] = (float)(z[k] / sum);",
                              "topk_weights[(size_t)t * K + k] = (float)z[k];")]),
    # LogFMT combine payload
    ("logfmt_lo_is_max", [("if (!any || l < lo)\n                    lo = l;", "if (!any || l > lo)\n                    lo = l;")]),
    ("logfmt_127_steps", [("const float inv = span > 0.0f ? 126.0f / span : 0.0f;",
                           "const float inv = span > 0.0f ? 127.0f / span : 0.0f;")]),
    ("logfmt_ties_away", [("int m = 1 + (int)nearbyintf(q);", "int m = 1 + (int)roundf(q);")]),
    ("logfmt_sign_dropped", [("code = (uint8_t)((v < 0.0f ? 0x80 : 0x00) | m);", "code = (uint8_t)m;")]),
    ("logfmt_zero_code_1", [("            uint8_t code = 0;\n", "            uint8_t code = 1;\n")]),
    ("logfmt_decode_from_m", [("const float d = lo + (float)(m - 1) * step;", "const float d = lo + (float)m * step;")]),
    ("logfmt_decode_127_steps", [("const float step = (hi - lo) / 126.0f;", "const float step = (hi - lo) / 127.0f;")]),
    ("logfmt_natural_log", [("float oracle_log2_rn(float a) { return (float)log2((double)a); }",
                             "float oracle_log2_rn(float a) { return (float)log((double)a); }")]),
    ("logfmt_log_truncated", [("float oracle_log2_rn(float a) { return (float)log2((double)a); }",
                               "float oracle_log2_rn(float a) { float l = (float)log2((double)a); double d = log2((double)a); return (double)l > d ? nextafterf(l, -1e30f) : l; }")]),
    ("combine_logfmt_header_of_block0", [("const float *hd = headers + ((size_t)r * (H / 128) + c / 128) * 2;",
                                          "const float *hd = headers + ((size_t)r * (H / 128)) * 2;")]),
    ("bias_row_of_token0", [(COMBINE_YR + COMBINE_FMA + "\n        }\n        add_bias_row(acc, bias ? bias + (size_t)t * H : NULL, H);",
                             COMBINE_YR + COMBINE_FMA + "\n        }\n        add_bias_row(acc, bias, H);")]),
]


def _build_and_run(name, edits, tmp):
    src = open(oracle.SOURCE).read()
    for old, new in edits:
        assert src.count(old) == 1, f"{name}: text to mutate must occur exactly once: {old!r}"
        src = src.replace(old, new)
    cpath = os.path.join(tmp, f"{name}.c")
    with open(cpath, "w") as f:
        f.write(src)
    so = oracle.build(cpath, os.path.join(tmp, f"lib_{name}.so"))
    res = subprocess.run([sys.executable, os.path.join(HERE, "mutant_runner.py"), so],
                         capture_output=True, text=True, timeout=600)
    return name, res.returncode, (res.stdout + res.stderr)[-400:]


def test_unmodified_oracle_passes_runner():
    res = subprocess.run([sys.executable, os.path.join(HERE, "mutant_runner.py"), oracle.get().path],
                         capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr


def test_every_planted_mistake_is_caught():
    with tempfile.TemporaryDirectory() as tmp:
        with concurrent.futures.ThreadPoolExecutor(max_workers=4) as pool:
            results = list(pool.map(lambda m: _build_and_run(m[0], m[1], tmp), MUTANTS))
    survivors = [(n, out) for n, rc, out in results if rc == 0]
    assert not survivors, f"mutants that passed every pin: {survivors}"
    for n, rc, out in results:
        print(n, "->", out.strip().splitlines()[-1] if out.strip() else f"exit {rc}")
