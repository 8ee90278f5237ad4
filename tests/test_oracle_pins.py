"""The CPU oracle against its pins (no GPU).

Each test names what pins the oracle: the DeepEP pages (a worked example on
the Lesson 14 routing table, the Ascend deep dive's bytes-per-pass figure),
brute-force enumeration, library routines (torch's bf16 and float8_e4m3fn
casts), closed forms, special cases and an error bound.
"""
import numpy as np
import pytest

import oracle
import pins
from cases import small_cases, with_dead_tokens
from combine_ep_layout_02_amd import workloads as W


@pytest.fixture(scope="module")
def o():
    return oracle.get()


def test_lesson_example(o):
    pins.pin_lesson_example(o)


def test_layout_bruteforce(o):
    pins.pin_layout_bruteforce(o)


def test_layout_bad_ids(o):
    pins.pin_layout_bad_ids(o)


def test_layout_invariants_full_size_routings(o):
    """The invariants on every workload's routing at its full token count
    (hidden shrunk to 128: the routing recipe does not depend on it)."""
    items = []
    for wid, w in W.WORKLOADS.items():
        ws = w.scaled(w.num_tokens, 128)
        inp = W.make_inputs(ws)
        items.append((inp, w.num_experts, w.num_ranks))
    pins.pin_layout_invariants(o, items)


def test_layout_edge_shapes(o):
    """N = 0, K = 1, every entry masked, R = 1, R = E, duplicate experts in a
    token (each entry its own slot, in k order; the rank counted once)."""
    empty = o.layout(np.zeros((0, 3), np.int64), 8, 4)
    assert empty["num_tokens_per_expert"].sum() == 0 and empty["num_tokens_per_rank"].sum() == 0
    assert empty["expert_offset"].tolist() == [0] * 9
    rng = np.random.default_rng(2)
    for (N, K, E, R) in [(33, 1, 8, 4), (20, 3, 6, 1), (20, 3, 6, 6)]:
        idx = rng.integers(-1, E, size=(N, K))
        pins.check_layout_invariants(o.layout(idx, E, R), idx, E, R)
    dead = -np.ones((9, 4), np.int64)
    lay = o.layout(dead, 8, 2)
    assert lay["num_tokens_per_rank"].tolist() == [0, 0] and np.all(lay["expert_slot"] == -1)
    dup = np.array([[3, 3, 1], [3, 0, 3], [2, 2, 2]], np.int64)
    lay = o.layout(dup, 4, 2)
    assert lay["expert_slot"].tolist() == [[0, 1, 0], [2, 0, 3], [0, 1, 2]]
    assert lay["num_tokens_per_rank"].tolist() == [2, 3]
    assert lay["rank_slot"].tolist() == [[0, 0], [1, 1], [-1, 2]]
    pins.check_layout_invariants(lay, dup, 4, 2)


def test_e4m3fn_structured(o):
    pins.pin_e4m3fn(o)


def test_e4m3fn_exhaustive_positive(o):
    pins.pin_e4m3fn_exhaustive_positive(o)


def test_bf16_rne(o):
    pins.pin_bf16(o)


def test_scales_closed_form(o):
    pins.pin_scales_closed_form(o)


def test_dequant_error_bound(o):
    pins.pin_dequant_bound(o)


def test_pack_payload_and_conservation(o):
    cases = []
    for w, inp in small_cases():
        cases.append((inp, w.num_experts, w.num_ranks, w.expert_capacity, w.use_fp8))
    pins.pin_pack(o, cases)
    pins.pin_pack_fp8_is_row_quantiser(o)


def test_combine_scalar_experts(o):
    cases = [(inp, w.num_experts, w.num_ranks, w.expert_capacity) for w, inp in small_cases()]
    pins.pin_combine_scalar_experts(o, cases)


def test_identity_expert(o):
    cases = []
    for w, inp in small_cases():
        cases.append((inp, w.num_experts, w.num_ranks, w.expert_capacity, w.use_fp8))
        cases.append((with_dead_tokens(inp), w.num_experts, w.num_ranks, w.expert_capacity, w.use_fp8))
    pins.pin_identity_expert(o, cases)


def test_lesson_dense_equivalence(o):
    pins.pin_lesson_dense(o, H=4)
    pins.pin_lesson_dense(o, H=128, seed=43)


def test_pages_bytes_per_pass(o):
    pins.pin_pages_pass_bytes(o)


def test_combine_random_rows_against_float64(o):
    """Combine of random expert rows against the same weighted sum in
    float64: within the tolerance plus the fp32 summation bound."""
    for w, inp in small_cases():
        idx, wt = inp["topk_idx"], inp["topk_weights"]
        E, R, S = w.num_experts, w.num_ranks, w.expert_capacity
        lay = o.layout(idx, E, R)
        y = pins.place_rows(inp["expert_rows"], idx, lay["expert_slot"], E, S)
        out, st = o.combine(y, idx, wt, lay["expert_slot"], E, S)
        assert st == 0
        ref = np.zeros(out.shape)
        mag = np.zeros(out.shape)
        rows = pins.bf16_to_f64(inp["expert_rows"])
        tt, kk = np.nonzero(idx >= 0)
        terms = wt[tt, kk].astype(np.float64)[:, None] * rows
        np.add.at(ref, tt, terms)
        np.add.at(mag, tt, np.abs(terms))
        K = idx.shape[1]
        pins.assert_combine_close(out, ref, abs_slack=K * 2.0 ** -24 * mag * 1.01)


def test_pow2_scales(o):
    pins.pin_pow2_scales(o)
    pins.pin_pow2_dequant_bound(o)


def test_ue8m0_packing(o):
    pins.pin_ue8m0_packing(o)


def _pack_cases(dead=False):
    cases = []
    for w, inp in small_cases():
        cases.append((inp, w.num_experts, w.num_ranks, w.expert_capacity, w.use_fp8))
        if dead:
            cases.append((with_dead_tokens(inp), w.num_experts, w.num_ranks, w.expert_capacity,
                          w.use_fp8))
    return cases


def test_receive_layouts_golden(o):
    pins.pin_receive_layouts_golden(o)


def test_expand_layout_matches_dense(o):
    pins.pin_expand_matches_dense(o, _pack_cases())


def test_normal_layout_matches_dense(o):
    pins.pin_normal_matches_dense(o, _pack_cases(dead=True))


def test_normal_combine_scalar_ranks(o):
    pins.pin_combine_normal_scalar_ranks(o, _pack_cases(dead=True))


def test_combine_bias_order(o):
    pins.pin_combine_bias_order(o)


def test_combine_bias_relations(o):
    pins.pin_combine_bias_relations(o, _pack_cases())


def test_backward_pair_adjoint(o):
    pins.pin_backward_pair_adjoint(o, _pack_cases(dead=True))


def test_gating_golden(o):
    pins.pin_gating_golden(o)


def test_gating_special_cases(o):
    pins.pin_gating_special_cases(o)


def test_gating_invariants(o):
    pins.pin_gating_invariants(o)
    pins.pin_gating_bad_args(o)


def test_gating_sum_rule(o):
    pins.pin_gating_sum_golden(o)
    pins.pin_gating_sum_special_cases(o)
    pins.pin_prefill_routing_is_sum_gating(o)


def test_logfmt(o):
    pins.pin_log2_rn_exhaustive(o)
    pins.pin_logfmt_golden(o)
    pins.pin_logfmt_roundtrip_bound(o)
    pins.pin_combine_logfmt_exact_cases(o)
