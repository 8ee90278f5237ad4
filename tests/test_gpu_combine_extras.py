"""GPU parity of the combine's epilogue bias and of the backward pair.

The shared expert's output added in the combine's epilogue (DeepEP Ascend
deep dive, "Combine: More Output, Same Cost") on all three combines, against
the oracle (bit-identical expected; the tolerance of the other combines is the
bar) and on the hand-worked rounding case that tells bias-last from
bias-first.  The backward pair of the DeepEP V1 Legacy guide §5.1 (dispatch's
backward is a combine, combine's backward a dispatch) as the exact adjoint
identity of ep_dispatch_normal and ep_combine_normal on integer-valued data.
"""
import numpy as np
import pytest
import torch

import oracle
import pins
from cases import small_cases
from combine_ep_layout_02_amd import ep
from combine_ep_layout_02_amd import workloads as W
from gpu_helpers import (POISON_X16, LayoutRun, dev, host, place_expert_rows, run_combine, say,
                         status_bits)
from test_gpu_receive_layouts import check_expand, check_normal

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def o():
    return oracle.get()


def _bias_rows(N, H, seed=31):
    rng = np.random.default_rng(seed)
    return W.bf16_bits(rng.standard_normal((N, H), dtype=np.float32))


def test_bias_order_hand_case(o):
    """Rows 2^-8, 2^-24, 2^-24 (weights 1) and a bias of 1 give 1 + 2^-7 when
    the bias is added after the sum (1.0 if it were added first)."""
    H, E = 1024, 3
    one, want = 0x3F80, 0x3F81
    vals = [0x3B80, 0x3380, 0x3380]  # bf16 bits of 2^-8, 2^-24, 2^-24
    idx = np.array([[0, 1, 2]], np.int64)
    bias = np.full((1, H), one, np.uint16)
    # per-expert layout
    shape = ep.make_shape(1, H, 3, E, 1, 1, 1, False)
    run = LayoutRun(shape, idx)
    y = torch.stack([torch.full((1, H), int(np.int16(np.uint16(v).view(np.int16))),
                                dtype=torch.int16, device="cuda") for v in vals])
    got, st = run_combine(shape, y, run.topk_idx, np.ones((1, 3), np.float32), run.expert_slot,
                          bias=bias)
    assert st == 0 and np.all(got == want), got[0, :4]
    # expand layout (alignment 1: rows 0, 1, 2)
    out = torch.full((1, H), int(POISON_X16), dtype=torch.int16, device="cuda")
    ep.ep_combine_expand(shape, y.reshape(3, H), run.topk_idx, dev(np.ones((1, 3), np.float32)),
                         run.expert_slot, run.expert_offset, out, bias=dev(bias))
    torch.cuda.synchronize()
    assert np.all(host(out) == want)
    # normal mode: three ranks, one row each
    shape3 = ep.make_shape(1, H, 3, E, 3, 1, 1, False)
    run3 = LayoutRun(shape3, idx)
    out.fill_(int(POISON_X16))
    ep.ep_combine_normal(shape3, y.reshape(3, 1, H), run3.rank_slot, None, out, bias=dev(bias))
    torch.cuda.synchronize()
    assert np.all(host(out) == want)


@pytest.mark.parametrize("case", range(5))
def test_combine_bias_small(o, case):
    w, inp = small_cases()[case]
    shape = ep.shape_of(w)
    run = LayoutRun(shape, inp["topk_idx"])
    lay = run.numpy()
    E, S, H, N = w.num_experts, w.expert_capacity, w.hidden, w.num_tokens
    y = place_expert_rows(inp["expert_rows"], inp["topk_idx"], lay["expert_slot"], E, S, H)
    s_or = max(1, int(lay["num_tokens_per_expert"].max()))
    y_or = pins.place_rows(inp["expert_rows"], inp["topk_idx"], lay["expert_slot"], E, s_or)
    bias = _bias_rows(N, H)
    say(f"ep_combine with bias {w.name}")
    got, st = run_combine(shape, y, run.topk_idx, inp["topk_weights"], run.expert_slot, bias=bias)
    want, st_or = o.combine(y_or, inp["topk_idx"], inp["topk_weights"], lay["expert_slot"], E, s_or,
                            bias=bias)
    assert st == st_or
    pins.assert_combine_close(got, pins.bf16_to_f64(want), "combine with bias")
    assert int((got != want).sum()) == 0
    check_expand(o, ep.shape_of(w, expert_alignment=16), inp, f"expand bias {w.name}",
                 y_rows=inp["expert_rows"], bias=bias)
    check_normal(o, shape, inp, f"normal bias {w.name}", bias=bias)


def test_combine_bias_full_size_prefill(o):
    w = W.WORKLOADS[3]
    inp = W.make_inputs(w, with_expert_rows=True)
    shape = ep.shape_of(w)
    run = LayoutRun(shape, inp["topk_idx"])
    lay = run.numpy()
    E, S, H, N = w.num_experts, w.expert_capacity, w.hidden, w.num_tokens
    y = place_expert_rows(inp["expert_rows"], inp["topk_idx"], lay["expert_slot"], E, S, H)
    s_or = max(1, int(lay["num_tokens_per_expert"].max()))
    y_or = pins.place_rows(inp["expert_rows"], inp["topk_idx"], lay["expert_slot"], E, s_or)
    bias = _bias_rows(N, H)
    say(f"ep_combine with bias {w.name}")
    got, st = run_combine(shape, y, run.topk_idx, inp["topk_weights"], run.expert_slot, bias=bias)
    want, _ = o.combine(y_or, inp["topk_idx"], inp["topk_weights"], lay["expert_slot"], E, s_or,
                        bias=bias)
    assert st == 0 and int((got != want).sum()) == 0


def _integer_bf16(rng, shape):
    return torch.from_numpy(rng.integers(-8, 9, size=shape).astype(np.float32)).to(
        torch.bfloat16).view(torch.int16)


@pytest.mark.parametrize("which", ["small_decode", "small_skewed", "full_prefill"])
def test_backward_pair_adjoint(o, which):
    """sum <dispatch_normal(x), g> == sum <x, combine_normal(g)> and the same
    for the weights (weight gradients zero where the receive side holds no
    weight), exactly, on the GPU."""
    if which == "full_prefill":
        w = W.WORKLOADS[3]
        inp = W.make_inputs(w.scaled(w.num_tokens, 1024))
    else:
        w, inp = small_cases()[1 if which == "small_decode" else 4]
    N, H, K, E, R = w.num_tokens, w.hidden, w.num_topk, w.num_experts, w.num_ranks
    M = w.num_max_dispatch_tokens_per_rank
    shape = ep.make_shape(N, H, K, E, R, M, w.expert_capacity, False)  # BF16: gradients
    run = LayoutRun(shape, inp["topk_idx"])
    lay = run.numpy()
    rng = np.random.default_rng(41)
    x = _integer_bf16(rng, (N, H)).cuda()
    wi = torch.from_numpy(rng.integers(-8, 9, size=(N, K)).astype(np.float32)).cuda()
    recv = torch.zeros((R, M, H), dtype=torch.int16, device="cuda")
    rti = torch.full((R, M, K), -1, dtype=torch.int64, device="cuda")
    rtw = torch.zeros((R, M, K), dtype=torch.float32, device="cuda")
    src = torch.full((R, M), -1, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    say(f"backward pair {which}: dispatch")
    ep.ep_dispatch_normal(shape, x, run.topk_idx, wi, run.rank_slot, recv, None, rti, rtw, src,
                          status)
    written = torch.zeros((R, M), dtype=torch.bool, device="cuda")
    for r in range(R):
        written[r, :int(lay["num_tokens_per_rank"][r])] = True
    g = (_integer_bf16(rng, (R, M, H)).cuda().view(torch.bfloat16).float() * written[:, :, None])
    g_bits = g.to(torch.bfloat16).view(torch.int16).contiguous()
    gw = torch.from_numpy(rng.integers(-8, 9, size=(R, M, K)).astype(np.float32)).cuda()
    gw = gw * ((rti >= 0) & written[:, :, None])
    out = torch.empty((N, H), dtype=torch.int16, device="cuda")
    cgw = torch.empty((N, K), dtype=torch.float32, device="cuda")
    say(f"backward pair {which}: combine")
    ep.ep_combine_normal(shape, g_bits, run.rank_slot, gw.contiguous(), out, cgw, status)
    torch.cuda.synchronize()
    assert status_bits(status) == 0
    recv_f = recv.view(torch.bfloat16).double() * written[:, :, None]
    lhs = float((recv_f * g.double()).sum())
    rhs = float((x.view(torch.bfloat16).double() * out.view(torch.bfloat16).double()).sum())
    assert lhs == rhs, (lhs, rhs)
    lw = float((rtw.double() * written[:, :, None] * gw.double()).sum())
    rw = float((wi.double() * cgw.double()).sum())
    assert lw == rw, (lw, rw)


def test_hip_graph_other_paths(o):
    """Gating, layout, expand pack and combine, normal pack and combine (with
    the bias) captured once in a HIP graph and replayed with new inputs
    copied into the captured buffers, eager work between replays; every
    replay equals an eager run on the same inputs and the oracle."""
    w = W.WORKLOADS[3].scaled(300, 512)
    N, H, K, E, R = w.num_tokens, w.hidden, w.num_topk, w.num_experts, w.num_ranks
    shape = ep.shape_of(w, expert_alignment=128)
    dev = torch.device("cuda")
    buf = ep.allocate(shape, dev, parts=("layout", "normal", "expand"))
    T = ep.expand_rows(shape)
    scores = torch.empty((N, E), dtype=torch.float32, device=dev)
    x = torch.empty((N, H), dtype=torch.int16, device=dev)
    y_exp = torch.empty((T, H), dtype=torch.int16, device=dev)
    y_nrm = torch.empty((R, w.num_max_dispatch_tokens_per_rank, H), dtype=torch.int16, device=dev)
    bias = torch.empty((N, H), dtype=torch.int16, device=dev)
    idx = torch.empty((N, K), dtype=torch.int64, device=dev)
    wts = torch.empty((N, K), dtype=torch.float32, device=dev)
    out_e = torch.empty((N, H), dtype=torch.int16, device=dev)
    out_n = torch.empty((N, H), dtype=torch.int16, device=dev)

    def step():
        ep.ep_group_limited_topk(shape, 8, 4, ep.EP_GATE_SUM_SIGMOID, scores, idx, wts)
        ep.ep_layout(shape, idx, buf["num_tokens_per_rank"], buf["num_tokens_per_expert"],
                     buf["is_token_in_rank"], buf["expert_slot"], buf["rank_slot"],
                     buf["expert_offset"], buf["workspace"], buf["status"])
        ep.ep_dispatch_expand(shape, x, idx, buf["expert_slot"], buf["expert_offset"],
                              buf["num_tokens_per_expert"], buf["recv_x_expand"],
                              buf["recv_scales_expand"], buf["recv_src_idx_expand"], buf["status"])
        ep.ep_combine_expand(shape, y_exp, idx, wts, buf["expert_slot"], buf["expert_offset"], out_e,
                             buf["status"], bias=bias)
        ep.ep_dispatch_normal(shape, x, idx, wts, buf["rank_slot"], buf["recv_x_normal"],
                              buf["recv_scales_normal"], buf["recv_topk_idx"],
                              buf["recv_topk_weights"], buf["recv_src_idx_normal"], buf["status"])
        ep.ep_combine_normal(shape, y_nrm, buf["rank_slot"], buf["recv_topk_weights"], out_n,
                             buf["combined_topk_weights"], buf["status"], bias=bias)

    def load(seed):
        rng = np.random.default_rng(seed)
        scores.copy_(torch.from_numpy(rng.standard_normal((N, E)).astype(np.float32)))
        x.copy_(torch.from_numpy(W.bf16_bits(rng.standard_normal((N, H), dtype=np.float32)).view(np.int16)))
        y_exp.copy_(torch.from_numpy(W.bf16_bits(rng.standard_normal((T, H), dtype=np.float32)).view(np.int16)))
        y_nrm.copy_(torch.from_numpy(W.bf16_bits(
            rng.standard_normal(tuple(y_nrm.shape), dtype=np.float32)).view(np.int16)))
        bias.copy_(torch.from_numpy(W.bf16_bits(rng.standard_normal((N, H), dtype=np.float32)).view(np.int16)))

    def snapshot():
        torch.cuda.synchronize()
        used = int(buf["expert_offset"][-1].item())
        return {"idx": idx.cpu().numpy(), "wts": wts.cpu().numpy(),
                "off": buf["expert_offset"].cpu().numpy(),
                "recv_e": buf["recv_x_expand"][:used].cpu().numpy(),
                "recv_n": buf["recv_x_normal"].cpu().numpy(),
                "cnt_r": buf["num_tokens_per_rank"].cpu().numpy(),
                "out_e": out_e.cpu().numpy(), "out_n": out_n.cpu().numpy(),
                "cw": buf["combined_topk_weights"].cpu().numpy()}

    load(3)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep, seed in enumerate((5, 5, 6, 7)):
        say(f"graph replay {rep} of the other paths (seed {seed})")
        load(seed)
        torch.cuda.synchronize()
        step()
        eager = snapshot()
        out_e.fill_(-1)
        out_n.fill_(-1)  # ordinary eager work between replays
        graph.replay()
        replay = snapshot()
        for key in eager:
            assert np.array_equal(eager[key].view(np.uint8), replay[key].view(np.uint8)), (rep, key)
        assert int(buf["status"].item()) == 0
        # and the oracle on this replay's inputs
        want_idx, _, _ = o.group_limited_topk(scores.cpu().numpy(), 8, 4, K,
                                             oracle.GATE_SUM_SIGMOID)
        assert np.array_equal(replay["idx"], want_idx)
        lay = o.layout(want_idx, E, R, alignment=128)
        assert np.array_equal(replay["off"], lay["expert_offset"])
        want_e, _ = o.combine_expand(y_exp.cpu().numpy().view(np.uint16), want_idx, replay["wts"],
                                     lay["expert_slot"], lay["expert_offset"],
                                     bias=bias.cpu().numpy().view(np.uint16))
        assert np.array_equal(replay["out_e"].view(np.uint16), want_e)
