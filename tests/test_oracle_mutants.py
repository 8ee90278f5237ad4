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
    ("fma_operands_swapped", [("acc[c] = fmaf(w, oracle_bf16_to_f32(yr[c]), acc[c]);",
                               "acc[c] = fmaf(w, acc[c], oracle_bf16_to_f32(yr[c]));")]),
    ("weight_of_first_k", [("float w = topk_weights[i];", "float w = topk_weights[(size_t)t * K];")]),
    ("combine_acc_negzero", [("            acc[c] = 0.0f;", "            acc[c] = -0.0f;")]),
    ("src_idx_is_k", [("recv_src_idx[row] = t;", "recv_src_idx[row] = k;")]),
    ("scales_row_stride", [("memcpy((float *)recv_scales + row * G, sc", "memcpy((float *)recv_scales + row, sc")]),
    ("dequant_wrong_block", [("float v = qv * scales[c / 128];", "float v = qv * scales[c % (H / 128)];")]),
    ("pow2_steps_past_equality", [("while (ldexp(448.0, e) < (double)ap)", "while (ldexp(448.0, e) <= (double)ap)")]),
    ("pow2_search_starts_high", [("    e -= 9;", "    e -= 7;")]),
    ("ue8m0_bias_128", [("(uint32_t)(ex[b] + 127) << (8 * (b % 4))", "(uint32_t)(ex[b] + 128) << (8 * (b % 4))")]),
    ("ue8m0_byte_order", [("<< (8 * (b % 4))", "<< (8 * (3 - b % 4))")]),
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
