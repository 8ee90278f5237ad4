"""GPU parity of the two other receive layouts against the CPU oracle.

Expand layout (DeepEP Ascend deep dive, "Dispatch's Three Phases", phase 1:
per-expert queues in one buffer, zero-padded to the expert alignment) and
normal mode (DeepEP V1 Legacy guide §5.1: one row per (token, rank), with
local expert ids and weights).  Same bar as the per-expert path: layout
offsets, bytes, scales, source indices, routing entries and weights are
bit-exact; combines are within 1 bf16 ulp or 8e-3 relative of the oracle and
are expected (and asserted) to be bit-identical.  Outputs start poisoned;
rows the kernels must not write are checked to still hold the poison.
"""
import numpy as np
import pytest
import torch

import oracle
import pins
from cases import small_cases
from combine_ep_layout_02_amd import ep
from combine_ep_layout_02_amd import workloads as W
from gpu_helpers import (POISON_I32, POISON_SCALE_BITS, POISON_SRC, POISON_X8, POISON_X16,
                         LayoutRun, dev, host, say, status_bits)

pytestmark = pytest.mark.gpu

POISON_W_BITS = 0x7FC0BEEF  # NaN pattern for float outputs, set through an int32 view


@pytest.fixture(scope="module")
def o():
    return oracle.get()


def first_diff(a, b):
    d = np.argwhere(np.asarray(a) != np.asarray(b))
    return None if d.size == 0 else (tuple(d[0]), np.asarray(a)[tuple(d[0])], np.asarray(b)[tuple(d[0])])


def _poisoned_rows(shape, rows):
    """Poisoned receive buffers of ``rows`` rows for the shape's payload."""
    H = shape.hidden
    if shape.use_fp8:
        rx = torch.full((rows, H), POISON_X8, dtype=torch.uint8, device="cuda")
        rs = torch.full((rows, ep.scale_row_elems(shape)), POISON_SCALE_BITS, dtype=torch.int32,
                        device="cuda")
        if shape.scale_format != ep.EP_SCALE_UE8M0:
            rs = rs.view(torch.float32)
    else:
        rx = torch.full((rows, H), int(POISON_X16), dtype=torch.int16, device="cuda")
        rs = None
    return rx, rs


def _bits(a):
    """Scales as raw 32-bit patterns (fp32 or UE8M0 words) for exact compares."""
    a = np.asarray(a)
    return a.view(np.uint32) if a.dtype in (np.float32, np.int32, np.uint32) else a


# ------------------------------------------------------------ expand layout

def check_layout_aligned(o, shape, topk_idx, name):
    A = max(shape.expert_alignment, 1)
    say(f"ep_layout {name} alignment={A} N={shape.num_tokens} E={shape.num_experts}")
    run = LayoutRun(shape, topk_idx)
    got = run.numpy()
    want = o.layout(topk_idx, shape.num_experts, shape.num_ranks, alignment=A)
    for key in ("num_tokens_per_expert", "expert_slot", "expert_offset", "rank_slot"):
        assert np.array_equal(got[key], want[key]), (name, key, first_diff(got[key], want[key]))
    return run, want


def check_expand(o, shape, inp, name, y_rows=None, bias=None):
    """Layout (aligned) + ep_dispatch_expand + ep_combine_expand against the
    oracle.  ``y_rows`` (one bf16 row per valid entry, (t, k) order) are the
    expert outputs for the combine; without them the combine is skipped."""
    run, lay = check_layout_aligned(o, shape, inp["topk_idx"], name)
    T = ep.expand_rows(shape)
    off = lay["expert_offset"].astype(np.int64)
    cnt = lay["num_tokens_per_expert"]
    used = int(off[-1])
    assert used <= T, "the aligned queues overflow the expand buffer"
    rx, rs = _poisoned_rows(shape, T)
    src = torch.full((T,), POISON_SRC, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    say(f"ep_dispatch_expand {name} fp8={shape.use_fp8} fmt={shape.scale_format} T={T} used={used}")
    ep.ep_dispatch_expand(shape, dev(inp["x_bits"]), run.topk_idx, run.expert_slot,
                          run.expert_offset, run.num_tokens_per_expert, rx, rs, src, status)
    torch.cuda.synchronize()
    want_x, want_s, want_src, st = o.pack_expand(inp["x_bits"], inp["topk_idx"], lay["expert_slot"],
                                                 off, cnt, max(used, 1), bool(shape.use_fp8),
                                                 scale_format=shape.scale_format)
    got_x = host(rx[:used])
    assert np.array_equal(got_x, want_x[:used]), (name, "recv_x", first_diff(got_x, want_x[:used]))
    got_src = host(src[:used])
    assert np.array_equal(got_src, want_src[:used]), (name, "recv_src_idx")
    if shape.use_fp8:
        got_s = _bits(host(rs[:used].view(torch.int32)))
        assert np.array_equal(got_s, _bits(want_s[:used])), (name, "recv_scales")
    # rows past the last queue are never written
    if used < T:
        poison = POISON_X8 if shape.use_fp8 else int(POISON_X16)
        assert not bool((rx[used:] != poison).any()), (name, "rows past the last queue written")
        assert not bool((src[used:] != POISON_SRC).any())
        if shape.use_fp8:
            assert not bool((rs[used:].view(torch.int32) != POISON_SCALE_BITS).any())
    assert status_bits(status) == st, (name, status_bits(status), st)
    if y_rows is None:
        return run, lay
    # combine over expert outputs placed at the expand rows (padding rows are
    # poisoned: the combine must not read them)
    idx, slot = inp["topk_idx"], lay["expert_slot"]
    valid = idx >= 0
    where = off[idx[valid]] + slot[valid].astype(np.int64)
    assert where.size == 0 or (where.min() >= 0 and where.max() < used)
    y_host = np.full((max(used, 1), shape.hidden), 0xA5A5, np.uint16)
    y_host[where] = y_rows
    y = torch.full((T, shape.hidden), int(POISON_X16), dtype=torch.int16, device="cuda")
    y[:max(used, 1)] = dev(y_host)
    out = torch.full((shape.num_tokens, shape.hidden), int(POISON_X16), dtype=torch.int16,
                     device="cuda")
    status.zero_()
    say(f"ep_combine_expand {name}")
    ep.ep_combine_expand(shape, y, run.topk_idx, dev(inp["topk_weights"]), run.expert_slot,
                         run.expert_offset, out, status, bias=None if bias is None else dev(bias))
    torch.cuda.synchronize()
    got = host(out)
    want, st2 = o.combine_expand(y_host, idx, inp["topk_weights"], slot, off, bias=bias)
    assert status_bits(status) == st2
    pins.assert_combine_close(got, pins.bf16_to_f64(want), f"{name} combine_expand")
    assert int((got != want).sum()) == 0, f"{name}: combine_expand not bit-identical"
    return run, lay


FMTS = [(ep.EP_SCALE_FP32, "fp32"), (ep.EP_SCALE_POW2, "pow2"), (ep.EP_SCALE_UE8M0, "ue8m0")]


@pytest.mark.parametrize("A", [0, 2, 128])
@pytest.mark.parametrize("case", range(5))
def test_expand_small(o, case, A):
    w, inp = small_cases()[case]
    for fmt, label in (FMTS if w.use_fp8 else FMTS[:1]):
        shape = ep.shape_of(w, fmt, expert_alignment=A)
        check_expand(o, shape, inp, f"small {w.name} A={A} {label}", y_rows=inp["expert_rows"])


@pytest.mark.parametrize("A", [1, 1024])
def test_layout_alignment_full_size(o, A):
    for wid, w in W.WORKLOADS.items():
        inp = W.make_inputs(w.scaled(w.num_tokens, 128))
        check_layout_aligned(o, ep.shape_of(w, expert_alignment=A), inp["topk_idx"], w.name)


def test_expand_full_size_prefill(o):
    """4,096 x 7,168 FP8, 256 experts, the Ascend page's alignment of 128."""
    w = W.WORKLOADS[3]
    inp = W.make_inputs(w, with_expert_rows=True)
    check_expand(o, ep.shape_of(w, expert_alignment=128), inp, f"full {w.name} A=128",
                 y_rows=inp["expert_rows"])


def _edge_inputs(N, H, K, E, seed=0, mask=0.0):
    rng = np.random.default_rng(seed)
    idx = np.argsort(rng.random((N, E)), axis=1)[:, :K].astype(np.int64) if K <= E else \
        rng.integers(0, E, size=(N, K))
    if mask:
        idx[rng.random((N, K)) < mask] = -1
    x = W.bf16_bits(rng.standard_normal((N, H), dtype=np.float32))
    wts = rng.random((N, K)).astype(np.float32)
    P = int((idx >= 0).sum())
    rows = W.bf16_bits(rng.standard_normal((P, H), dtype=np.float32))
    return {"x_bits": x, "topk_idx": idx, "topk_weights": wts, "expert_rows": rows}


EXPAND_EDGE = [
    ("N=0", dict(N=0, H=256, K=4, E=16, R=4, use_fp8=True, A=128)),
    ("N=1 K=1 A=1024", dict(N=1, H=128, K=1, E=8, R=2, use_fp8=True, A=1024)),
    ("all masked", dict(N=70, H=256, K=3, E=8, R=4, use_fp8=True, A=16, mask=1.0)),
    ("ragged bf16 H=520 A=3", dict(N=257, H=520, K=5, E=32, R=8, use_fp8=False, A=3, mask=0.05)),
    ("E=1024 A=128", dict(N=600, H=128, K=8, E=1024, R=64, use_fp8=True, A=128)),
    ("K>E repeats A=8", dict(N=200, H=1152, K=12, E=8, R=4, use_fp8=True, A=8)),
]


@pytest.mark.parametrize("name,kw", EXPAND_EDGE, ids=[e[0] for e in EXPAND_EDGE])
def test_expand_edges(o, name, kw):
    kw = dict(kw)
    A, R, use_fp8 = kw.pop("A"), kw.pop("R"), kw.pop("use_fp8")
    N, H, K, E = kw["N"], kw["H"], kw["K"], kw["E"]
    inp = _edge_inputs(N, H, K, E, mask=kw.get("mask", 0.0))
    M = max(N, 1)
    for fmt, label in (FMTS if use_fp8 else FMTS[:1]):
        shape = ep.make_shape(N, H, K, E, R, M, M * max(1, -(-K // E)), use_fp8, fmt, A)
        check_expand(o, shape, inp, f"{name} {label}", y_rows=inp["expert_rows"])


def test_expand_slot_outside_queue_is_skipped_and_reported(o):
    """A slot past its expert's queue (here: a corrupted handle) is skipped by
    pack and combine and reported as EP_STATUS_BAD_SLOT, as in the oracle."""
    N, H, K, E, R, A = 64, 256, 4, 16, 4, 8
    inp = _edge_inputs(N, H, K, E)
    shape = ep.make_shape(N, H, K, E, R, N, N, True, 0, A)
    run, lay = check_layout_aligned(o, shape, inp["topk_idx"], "corrupt slot")
    slot = lay["expert_slot"].copy()
    slot[3, 1] += 1000  # past the queue
    slot[5, 0] = -3     # negative
    run.expert_slot.copy_(dev(slot))
    T = ep.expand_rows(shape)
    off, cnt = lay["expert_offset"], lay["num_tokens_per_expert"]
    rx, rs = _poisoned_rows(shape, T)
    src = torch.full((T,), POISON_SRC, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ep.ep_dispatch_expand(shape, dev(inp["x_bits"]), run.topk_idx, run.expert_slot,
                          run.expert_offset, run.num_tokens_per_expert, rx, rs, src, status)
    torch.cuda.synchronize()
    wx, ws, wsrc, st = o.pack_expand(inp["x_bits"], inp["topk_idx"], slot, off, cnt, T, True,
                                     fill=POISON_X8)
    assert st == ep.EP_STATUS_BAD_SLOT and status_bits(status) == st
    used = int(off[-1])
    assert np.array_equal(host(rx[:used]), wx[:used])
    assert np.array_equal(host(src[:used]), np.where(wsrc[:used] == -2, POISON_SRC, wsrc[:used]))


# -------------------------------------------------------------- normal mode

def check_normal(o, shape, inp, name, with_weights=True, rank_slot_override=None, bias=None):
    """Layout + ep_dispatch_normal + ep_combine_normal against the oracle."""
    run = LayoutRun(shape, inp["topk_idx"])
    lay = run.numpy()
    want_lay = o.layout(inp["topk_idx"], shape.num_experts, shape.num_ranks)
    for key in ("rank_slot", "num_tokens_per_rank", "is_token_in_rank"):
        assert np.array_equal(lay[key], want_lay[key]), (name, key)
    rank_slot = lay["rank_slot"] if rank_slot_override is None else rank_slot_override
    if rank_slot_override is not None:
        run.rank_slot.copy_(dev(rank_slot))
    N, H, K, R = shape.num_tokens, shape.hidden, shape.num_topk, shape.num_ranks
    M = shape.num_max_dispatch_tokens_per_rank
    rows = R * M
    rx, rs = _poisoned_rows(shape, rows)
    rti = torch.full((rows, K), -7, dtype=torch.int64, device="cuda")
    rtw = torch.full((rows, K), POISON_W_BITS, dtype=torch.int32, device="cuda").view(torch.float32)
    src = torch.full((rows,), POISON_SRC, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    w = dev(inp["topk_weights"]) if with_weights else None
    say(f"ep_dispatch_normal {name} fp8={shape.use_fp8} fmt={shape.scale_format} R={R} M={M}")
    ep.ep_dispatch_normal(shape, dev(inp["x_bits"]), run.topk_idx, w, run.rank_slot, rx, rs, rti,
                          rtw if with_weights else None, src, status)
    torch.cuda.synchronize()
    want = o.dispatch_normal(inp["x_bits"], inp["topk_idx"],
                             inp["topk_weights"] if with_weights else None, rank_slot,
                             shape.num_experts, R, M, bool(shape.use_fp8),
                             scale_format=shape.scale_format)
    assert status_bits(status) == want["status"], (name, status_bits(status), want["status"])
    cnt = lay["num_tokens_per_rank"]
    gx, gsrc, gti = host(rx).reshape(R, M, H), host(src).reshape(R, M), host(rti).reshape(R, M, K)
    gtw = host(rtw.view(torch.int32)).reshape(R, M, K)
    gs = host(rs.view(torch.int32)).reshape(R, M, -1) if shape.use_fp8 else None
    poison = POISON_X8 if shape.use_fp8 else np.uint16(0xA5A5)
    for r in range(R):
        col = rank_slot[:, r] if N else np.zeros(0, np.int32)
        wr = np.sort(col[(col >= 0) & (col < M)]).astype(np.int64)  # rows written at rank r
        assert wr.size <= M
        assert np.array_equal(gx[r, wr], want["recv_x"][r, wr]), (name, r, "recv_x")
        assert np.array_equal(gsrc[r, wr], want["recv_src_idx"][r, wr]), (name, r, "src")
        assert np.array_equal(gti[r, wr], want["recv_topk_idx"][r, wr]), (name, r, "topk_idx")
        if with_weights:
            assert np.array_equal(gtw[r, wr].view(np.uint32),
                                  want["recv_topk_weights"][r, wr].view(np.uint32)), (name, r, "w")
        if shape.use_fp8:
            assert np.array_equal(_bits(gs[r, wr]), _bits(want["recv_scales"][r, wr])), (name, r)
        # every other row keeps the poison
        rest = np.setdiff1d(np.arange(M), wr)
        assert np.all(gx[r, rest] == poison) and np.all(gsrc[r, rest] == POISON_SRC)
        assert np.all(gti[r, rest] == -7) and np.all(gtw[r, rest] == POISON_W_BITS)
        if shape.use_fp8:
            assert np.all(gs[r, rest].view(np.uint32) == POISON_SCALE_BITS)
    if not with_weights:
        assert np.all(gtw == POISON_W_BITS), "weights written although none were given"
    # combine: random bf16 rows for each received token, rows past the count poisoned
    rng = np.random.default_rng(99)
    y_host = np.full((R, M, H), 0xA5A5, np.uint16)
    for r in range(R):
        c = min(int(cnt[r]), M)
        y_host[r, :c] = W.bf16_bits(rng.standard_normal((c, H), dtype=np.float32))
    out = torch.full((N, H), int(POISON_X16), dtype=torch.int16, device="cuda")
    cw = torch.full((N, K), POISON_W_BITS, dtype=torch.int32, device="cuda").view(torch.float32)
    status.zero_()
    say(f"ep_combine_normal {name}")
    ep.ep_combine_normal(shape, dev(y_host), run.rank_slot, rtw if with_weights else None, out,
                         cw if with_weights else None, status,
                         bias=None if bias is None else dev(bias))
    torch.cuda.synchronize()
    got = host(out)
    want_out, want_cw, st = o.combine_normal(y_host, rank_slot,
                                             want["recv_topk_weights"] if with_weights else None,
                                             bias=bias)
    assert status_bits(status) == st
    pins.assert_combine_close(got, pins.bf16_to_f64(want_out), f"{name} combine_normal")
    assert int((got != want_out).sum()) == 0, f"{name}: combine_normal not bit-identical"
    if with_weights:
        assert np.array_equal(host(cw).view(np.uint32), want_cw.view(np.uint32)), (name, "weights")
    else:
        assert np.all(host(cw.view(torch.int32)) == POISON_W_BITS)


@pytest.mark.parametrize("case", range(5))
def test_normal_small(o, case):
    w, inp = small_cases()[case]
    for fmt, label in (FMTS if w.use_fp8 else FMTS[:1]):
        check_normal(o, ep.shape_of(w, fmt), inp, f"small {w.name} {label}")
    check_normal(o, ep.shape_of(w), inp, f"small {w.name} no weights", with_weights=False)


@pytest.mark.parametrize("wid", [3, 5])
def test_normal_full_size(o, wid):
    w = W.WORKLOADS[wid]
    inp = W.make_inputs(w)
    check_normal(o, ep.shape_of(w), inp, f"full {w.name}")


NORMAL_EDGE = [
    ("N=0", dict(N=0, H=256, K=4, E=16, R=4, use_fp8=True)),
    ("N=1 K=1", dict(N=1, H=128, K=1, E=8, R=2, use_fp8=True)),
    ("all masked", dict(N=70, H=256, K=3, E=8, R=4, use_fp8=True, mask=1.0)),
    ("R=1", dict(N=300, H=128, K=4, E=16, R=1, use_fp8=True)),
    ("R=E=64", dict(N=300, H=256, K=6, E=64, R=64, use_fp8=True, mask=0.2)),
    ("ragged bf16 H=520", dict(N=257, H=520, K=5, E=32, R=8, use_fp8=False, mask=0.05)),
    ("K=32 E=1024 R=64", dict(N=300, H=128, K=32, E=1024, R=64, use_fp8=False, mask=0.1)),
    ("K>E repeats", dict(N=200, H=1152, K=12, E=8, R=4, use_fp8=True)),
    ("N<M", dict(N=50, H=256, K=8, E=64, R=8, use_fp8=True, M=64)),
]


@pytest.mark.parametrize("name,kw", NORMAL_EDGE, ids=[e[0] for e in NORMAL_EDGE])
def test_normal_edges(o, name, kw):
    kw = dict(kw)
    R, use_fp8 = kw.pop("R"), kw.pop("use_fp8")
    N, H, K, E = kw["N"], kw["H"], kw["K"], kw["E"]
    M = kw.get("M", max(N, 1))
    inp = _edge_inputs(N, H, K, E, mask=kw.get("mask", 0.0))
    for fmt, label in (FMTS if use_fp8 else FMTS[:1]):
        shape = ep.make_shape(N, H, K, E, R, M, M * max(1, -(-K // E)), use_fp8, fmt)
        check_normal(o, shape, inp, f"{name} {label}")


def test_normal_bad_ids_and_slots_are_reported(o):
    """Expert ids outside [-1, E) read as -1 (and set EP_STATUS_BAD_EXPERT_ID
    for tokens that are written); a rank slot >= M (a corrupted handle) is
    skipped by dispatch and combine and sets EP_STATUS_BAD_SLOT."""
    N, H, K, E, R = 96, 256, 4, 16, 4
    inp = _edge_inputs(N, H, K, E, seed=5)
    inp["topk_idx"][7, 2] = E + 3
    inp["topk_idx"][11, 0] = -5
    shape = ep.make_shape(N, H, K, E, R, N, N, True)
    lay = o.layout(inp["topk_idx"], E, R)
    rs = lay["rank_slot"].copy()
    r0 = int(np.nonzero(rs[20] >= 0)[0][0])
    rs[20, r0] = N + 5  # >= M
    check_normal(o, shape, inp, "bad ids", rank_slot_override=rs)


@pytest.mark.parametrize("mode", ["normal", "expand"])
def test_receive_layout_step_hip_graph_replay(mode):
    """The normal-mode and expand steps (layout, dispatch, combine) captured
    once in a HIP graph and replayed with new routings, inputs and expert
    outputs copied into the captured buffers, eager work in between; every
    replay must reproduce an eager run of the same inputs exactly."""
    base = W.WORKLOADS[2].scaled(300, 1024)
    shape = ep.shape_of(base, expert_alignment=128 if mode == "expand" else 0)
    N, H, K, E, R, M = (shape.num_tokens, shape.hidden, shape.num_topk, shape.num_experts,
                        shape.num_ranks, shape.num_max_dispatch_tokens_per_rank)
    d = torch.device("cuda")
    buf = ep.allocate(shape, d, parts=("layout", "combine", mode))
    idx = torch.empty((N, K), dtype=torch.int64, device=d)
    wts = torch.empty((N, K), dtype=torch.float32, device=d)
    x = torch.empty((N, H), dtype=torch.int16, device=d)
    if mode == "normal":
        y = torch.empty((R, M, H), dtype=torch.int16, device=d)
        rw = torch.empty((R, M, K), dtype=torch.float32, device=d)
        keys = ("recv_x_normal", "recv_scales_normal", "recv_topk_idx", "recv_topk_weights",
                "recv_src_idx_normal", "combined_x", "combined_topk_weights", "rank_slot",
                "num_tokens_per_rank")
    else:
        y = torch.empty((ep.expand_rows(shape), H), dtype=torch.int16, device=d)
        rw = None
        keys = ("recv_x_expand", "recv_scales_expand", "recv_src_idx_expand", "combined_x",
                "expert_slot", "expert_offset", "num_tokens_per_expert")

    def step():
        ep.ep_layout(shape, idx, buf["num_tokens_per_rank"], buf["num_tokens_per_expert"],
                     buf["is_token_in_rank"], buf["expert_slot"], buf["rank_slot"],
                     buf["expert_offset"], buf["workspace"], buf["status"])
        if mode == "normal":
            ep.ep_dispatch_normal(shape, x, idx, wts, buf["rank_slot"], buf["recv_x_normal"],
                                  buf["recv_scales_normal"], buf["recv_topk_idx"],
                                  buf["recv_topk_weights"], buf["recv_src_idx_normal"], buf["status"])
            ep.ep_combine_normal(shape, y, buf["rank_slot"], rw, buf["combined_x"],
                                 buf["combined_topk_weights"], buf["status"])
        else:
            ep.ep_dispatch_expand(shape, x, idx, buf["expert_slot"], buf["expert_offset"],
                                  buf["num_tokens_per_expert"], buf["recv_x_expand"],
                                  buf["recv_scales_expand"], buf["recv_src_idx_expand"], buf["status"])
            ep.ep_combine_expand(shape, y, idx, wts, buf["expert_slot"], buf["expert_offset"],
                                 buf["combined_x"], buf["status"])

    def load(seed):
        inp = W.make_inputs(base, seed=seed)
        idx.copy_(torch.from_numpy(inp["topk_idx"]))
        wts.copy_(torch.from_numpy(inp["topk_weights"]))
        x.copy_(torch.from_numpy(inp["x_bits"].view(np.int16)))
        g = torch.Generator(device=d)
        g.manual_seed(seed)
        y.copy_(torch.randn(y.shape, dtype=torch.bfloat16, device=d, generator=g).view(torch.int16))
        if rw is not None:
            rw.copy_(torch.rand(rw.shape, dtype=torch.float32, device=d, generator=g))

    def snapshot():
        torch.cuda.synchronize()
        return {k: buf[k].view(torch.uint8).cpu().numpy().copy() for k in keys if buf[k] is not None}

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
        say(f"{mode} graph replay {rep} (seed {seed})")
        load(seed)
        torch.cuda.synchronize()
        step()  # eager reference on the same inputs
        eager = snapshot()
        buf["combined_x"].fill_(-1)  # ordinary eager work between replays
        buf["num_tokens_per_rank" if mode == "normal" else "num_tokens_per_expert"].fill_(-1)
        graph.replay()
        replay = snapshot()
        for k in eager:
            assert np.array_equal(eager[k], replay[k]), (mode, rep, k)
    assert int(buf["status"].item()) == 0
