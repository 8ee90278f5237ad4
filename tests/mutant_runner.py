"""Run the oracle pins against one build of the oracle library.

Usage: python tests/mutant_runner.py /path/to/libep_oracle_variant.so

Exit status 0: every pin passed.  1: a pin failed (its name is printed).
Used by test_oracle_mutants.py, which runs it in a child process per planted
mistake so that a variant that crashes cannot take the test session down.
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path[:0] = [os.path.dirname(HERE), HERE]

import oracle  # noqa: E402
import pins  # noqa: E402
from cases import small_cases, with_dead_tokens  # noqa: E402


def main(path: str) -> int:
    o = oracle.Oracle(path)
    sc = small_cases()
    pack_cases = [(inp, w.num_experts, w.num_ranks, w.expert_capacity, w.use_fp8) for w, inp in sc]
    ident_cases = pack_cases + [(with_dead_tokens(inp), E, R, S, f8) for (inp, E, R, S, f8) in pack_cases]
    comb_cases = [(inp, w.num_experts, w.num_ranks, w.expert_capacity) for w, inp in sc]
    inv_cases = [(inp, w.num_experts, w.num_ranks) for w, inp in sc]
    steps = [
        ("lesson_example", lambda: pins.pin_lesson_example(o)),
        ("bf16", lambda: pins.pin_bf16(o)),
        ("e4m3fn", lambda: pins.pin_e4m3fn(o)),
        ("scales_closed_form", lambda: pins.pin_scales_closed_form(o)),
        ("dequant_bound", lambda: pins.pin_dequant_bound(o)),
        ("layout_bad_ids", lambda: pins.pin_layout_bad_ids(o)),
        ("layout_invariants", lambda: pins.pin_layout_invariants(o, inv_cases)),
        ("pack", lambda: pins.pin_pack(o, pack_cases)),
        ("pack_fp8_row", lambda: pins.pin_pack_fp8_is_row_quantiser(o)),
        ("combine_scalar", lambda: pins.pin_combine_scalar_experts(o, comb_cases)),
        ("identity", lambda: pins.pin_identity_expert(o, ident_cases)),
        ("lesson_dense", lambda: pins.pin_lesson_dense(o, H=4)),
        ("pages_bytes", lambda: pins.pin_pages_pass_bytes(o)),
        ("pow2_scales", lambda: pins.pin_pow2_scales(o)),
        ("pow2_dequant_bound", lambda: pins.pin_pow2_dequant_bound(o)),
        ("ue8m0_packing", lambda: pins.pin_ue8m0_packing(o)),
        ("receive_layouts_golden", lambda: pins.pin_receive_layouts_golden(o)),
        ("expand_matches_dense", lambda: pins.pin_expand_matches_dense(o, pack_cases)),
        ("normal_matches_dense", lambda: pins.pin_normal_matches_dense(o, ident_cases)),
        ("combine_normal_scalar", lambda: pins.pin_combine_normal_scalar_ranks(o, ident_cases)),
        ("combine_bias_order", lambda: pins.pin_combine_bias_order(o)),
        ("combine_bias_relations", lambda: pins.pin_combine_bias_relations(o, pack_cases)),
        ("backward_pair_adjoint", lambda: pins.pin_backward_pair_adjoint(o, ident_cases)),
        ("gating_golden", lambda: pins.pin_gating_golden(o)),
        ("gating_special_cases", lambda: pins.pin_gating_special_cases(o)),
        ("gating_invariants", lambda: pins.pin_gating_invariants(o)),
        ("gating_sum_golden", lambda: pins.pin_gating_sum_golden(o)),
        ("gating_sum_special_cases", lambda: pins.pin_gating_sum_special_cases(o)),
        ("gating_bad_args", lambda: pins.pin_gating_bad_args(o)),
        ("log2_rn_exhaustive", lambda: pins.pin_log2_rn_exhaustive(o)),
        ("logfmt_golden", lambda: pins.pin_logfmt_golden(o)),
        ("logfmt_roundtrip_bound", lambda: pins.pin_logfmt_roundtrip_bound(o)),
        ("combine_logfmt", lambda: pins.pin_combine_logfmt_exact_cases(o)),
        ("layout_bruteforce", lambda: pins.pin_layout_bruteforce(o)),
    ]
    for name, fn in steps:
        try:
            fn()
        except AssertionError as exc:
            print(f"FAILED {name}: {str(exc)[:200]}")
            return 1
    print("ALL PINS PASSED")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1]))
