"""GPU parity of ep_layout_dispatch (layout and per-expert pack in one call)
against the CPU oracle's layout and pack.

Bar: the same as ep_layout and ep_dispatch separately -- every layout output,
FP8 byte, scale, BF16 row and recv_src_idx bit-exact, rows past each expert's
count still poisoned, and the status word equal to the oracle's layout and
pack bits together.  Up to 256 tokens the call is one fused launch; up to
1,024 the layout's count kernel and one fused launch that adds the earlier
count blocks' histograms; above that a kernel that ranks each 256-token block
on its own and a pack (one block per token) that adds the earlier blocks'
counts.  The cases step across both boundaries; the workspace starts
poisoned."""
import numpy as np
import pytest
import torch

import oracle
from cases import small_cases
from combine_ep_layout_02_amd import ep
from combine_ep_layout_02_amd import workloads as W
from gpu_helpers import (POISON_I32, POISON_SCALE_BITS, POISON_SRC, POISON_U8, POISON_X8,
                         POISON_X16, dev, gather_rows, host, say, status_bits,
                         unwritten_rows_intact, written_rows)

pytestmark = pytest.mark.gpu

LAYOUT_KEYS = ("num_tokens_per_rank", "num_tokens_per_expert", "is_token_in_rank", "expert_slot",
               "rank_slot", "expert_offset")


@pytest.fixture(scope="module")
def o():
    return oracle.get()


def oracle_capacity(counts, S):
    top = int(counts.max()) if counts.size else 0
    return S if top > S else max(1, top)


def launch_fused(shape, x_bits, topk_idx, topk_offset=0, workspace=None):
    """Enqueue one ep_layout_dispatch call on poisoned outputs (a poisoned
    workspace of its own unless one is given).  With topk_offset > 0 the ids
    sit that many int64 into their buffer (an 8-byte aligned base that is not
    16-byte aligned when the offset is odd)."""
    N, H, K, E, R, S = (shape.num_tokens, shape.hidden, shape.num_topk, shape.num_experts,
                        shape.num_ranks, shape.expert_capacity)
    full = lambda n, v, dt: torch.full((n,), v, dtype=dt, device="cuda")
    ids = np.concatenate([np.zeros(topk_offset, np.int64), np.asarray(topk_idx, np.int64).reshape(-1)])
    ids_dev = dev(ids)[topk_offset:].view(N, K)
    out = {
        "num_tokens_per_rank": full(R, POISON_I32, torch.int32),
        "num_tokens_per_expert": full(E, POISON_I32, torch.int32),
        "is_token_in_rank": full(N * R, POISON_U8, torch.uint8).view(N, R),
        "expert_slot": full(N * K, POISON_I32, torch.int32).view(N, K),
        "rank_slot": full(N * R, POISON_I32, torch.int32).view(N, R),
        "expert_offset": full(E + 1, POISON_I32, torch.int32),
    }
    need = ep.ep_query_sizes(shape)["layout_workspace"]
    if workspace is None and need:
        workspace = full(-(-need // 4), POISON_I32, torch.int32)
    if shape.use_fp8:
        recv_x = torch.full((E, S, H), POISON_X8, dtype=torch.uint8, device="cuda")
        recv_scales = torch.full((E, S, ep.scale_row_elems(shape)), POISON_SCALE_BITS,
                                 dtype=torch.int32, device="cuda")
        if shape.scale_format != ep.EP_SCALE_UE8M0:
            recv_scales = recv_scales.view(torch.float32)
    else:
        recv_x = torch.full((E, S, H), int(POISON_X16), dtype=torch.int16, device="cuda")
        recv_scales = None
    recv_src_idx = torch.full((E, S), POISON_SRC, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    x = dev(x_bits) if N else torch.empty((0, H), dtype=torch.int16, device="cuda")
    ep.ep_layout_dispatch(shape, ids_dev, x, out["num_tokens_per_rank"], out["num_tokens_per_expert"],
                          out["is_token_in_rank"], out["expert_slot"], out["rank_slot"],
                          out["expert_offset"], workspace, recv_x, recv_scales, recv_src_idx, status)
    return out, recv_x, recv_scales, recv_src_idx, status


def run_fused(shape, x_bits, topk_idx, topk_offset=0, workspace=None):
    res = launch_fused(shape, x_bits, topk_idx, topk_offset, workspace)
    torch.cuda.synchronize()
    return res


def check_fused(o, shape, x_bits, topk_idx, name, topk_offset=0, workspace=None, result=None):
    """Every output of one call against the oracle; `result` is a call
    already made (launch_fused, then a synchronize), else one is made here."""
    N, H, E, R, S = shape.num_tokens, shape.hidden, shape.num_experts, shape.num_ranks, \
        shape.expert_capacity
    say(f"ep_layout_dispatch {name} N={N} H={H} K={shape.num_topk} E={E} R={R} S={S} "
        f"fp8={shape.use_fp8} scale_format={shape.scale_format}")
    if result is None:
        result = run_fused(shape, x_bits, topk_idx, topk_offset, workspace)
    out, recv_x, recv_scales, recv_src_idx, status = result
    lay = o.layout(topk_idx, E, R, alignment=max(shape.expert_alignment, 1))
    for key in LAYOUT_KEYS:
        got = host(out[key])
        assert np.array_equal(got, lay[key]), (name, key)
    counts = lay["num_tokens_per_expert"]
    s_or = oracle_capacity(counts, S)
    rx, rs, src, st = o.pack(x_bits, topk_idx, lay["expert_slot"], E, s_or, bool(shape.use_fp8),
                             scale_format=shape.scale_format)
    rows_gpu, rows_or = written_rows(counts, S), written_rows(counts, s_or)
    assert np.array_equal(gather_rows(recv_x, rows_gpu), rx.reshape(E * s_or, H)[rows_or]), (name, "recv_x")
    assert np.array_equal(gather_rows(recv_src_idx, rows_gpu), src.reshape(-1)[rows_or]), (name, "src")
    if shape.use_fp8:
        got_sc = gather_rows(recv_scales.view(torch.int32), rows_gpu)
        want_sc = rs.reshape(E * s_or, rs.shape[-1])[rows_or].view(np.int32)
        assert np.array_equal(got_sc, want_sc), (name, "recv_scales")
        assert unwritten_rows_intact(recv_x, counts, POISON_X8)
        assert unwritten_rows_intact(recv_scales.view(torch.int32), counts, POISON_SCALE_BITS)
    else:
        assert unwritten_rows_intact(recv_x, counts, int(POISON_X16))
    assert unwritten_rows_intact(recv_src_idx, counts, POISON_SRC)
    assert status_bits(status) == (lay["status"] | st), (name, status_bits(status), lay["status"], st)
    return status_bits(status)


def _random(N, H, K, E, R, seed, mask=0.0, repeats=False):
    rng = np.random.default_rng(seed)
    if repeats:
        idx = rng.integers(0, E, size=(N, K)).astype(np.int64)
    else:
        idx = np.argsort(rng.random((N, E)), axis=1)[:, :K].astype(np.int64)
    if mask:
        idx[rng.random((N, K)) < mask] = -1
    x = W.bf16_bits(rng.standard_normal((N, H), dtype=np.float32))
    return x, idx


@pytest.mark.parametrize("case", range(5))
def test_fused_small_cases(o, case):
    w, inp = small_cases()[case]
    check_fused(o, ep.shape_of(w), inp["x_bits"], inp["topk_idx"], f"small {w.name}")


@pytest.mark.parametrize("fmt", [ep.EP_SCALE_FP32, ep.EP_SCALE_POW2, ep.EP_SCALE_UE8M0],
                         ids=["fp32", "pow2", "ue8m0"])
def test_fused_decode_full_size(o, fmt):
    """128 tokens x 7,168, top-8 of 256 experts over 8 ranks, S = 1,024."""
    w = W.WORKLOADS[2]
    inp = W.make_inputs(w)
    check_fused(o, ep.shape_of(w, fmt), inp["x_bits"], inp["topk_idx"], f"full {w.name}")


@pytest.mark.parametrize("fmt", [ep.EP_SCALE_FP32, ep.EP_SCALE_POW2, ep.EP_SCALE_UE8M0],
                         ids=["fp32", "pow2", "ue8m0"])
def test_fused_prefill_1024_tokens(o, fmt):
    """The prefill routing (group-limited top-8 of 256 experts, 8 ranks) at
    1,024 tokens x 7,168, the largest batch of the count-kernel form."""
    w = W.WORKLOADS[3].scaled(1024, 7168)
    inp = W.make_inputs(w)
    check_fused(o, ep.shape_of(w, fmt), inp["x_bits"], inp["topk_idx"], f"prefill {w.name}")


EDGE = [
    # name, N, H, K, E, R, fp8, extra
    ("N=0", 0, 256, 4, 16, 4, True, {}),
    ("N=1 K=1", 1, 128, 1, 8, 2, True, {}),
    ("N=1 bf16 H=8", 1, 8, 2, 4, 2, False, {}),
    ("R=1", 200, 128, 4, 16, 1, True, {}),
    ("R=E=64 masked", 250, 256, 6, 64, 64, True, dict(mask=0.2)),
    ("odd K=5 bf16 H=520", 256, 520, 5, 32, 8, False, dict(mask=0.05)),
    ("N=256 (largest single launch)", 256, 1152, 8, 256, 8, True, {}),
    ("N=257 (count kernel + fused)", 257, 1152, 8, 256, 8, True, {}),
    ("N=513 R=1", 513, 128, 4, 16, 1, True, {}),
    ("N=600 R=E=64 masked", 600, 256, 6, 64, 64, True, dict(mask=0.2)),
    ("N=700 K=32 E=1024 R=64", 700, 128, 32, 1024, 64, False, dict(mask=0.1)),
    ("N=800 H=9216: three chunks per wave", 800, 9216, 8, 64, 8, True, {}),
    ("N=900 repeats K=12 E=8", 900, 128, 12, 8, 4, True, dict(repeats=True)),
    ("N=1000 K=16 E=256 R=32", 1000, 256, 16, 256, 32, True, dict(mask=0.1)),
    ("N=150 K=10 bf16", 150, 520, 10, 64, 8, False, {}),
    ("N=1024 odd K=5 bf16 H=520", 1024, 520, 5, 32, 8, False, dict(mask=0.05)),
    ("N=1025 (local ranks and pack)", 1025, 1152, 8, 256, 8, True, {}),
    ("N=1100 K=1", 1100, 256, 1, 32, 8, True, {}),
    ("N=1200 R=1", 1200, 128, 4, 16, 1, True, {}),
    ("N=1300 all masked", 1300, 256, 4, 16, 4, True, dict(mask=1.0)),
    ("N=1500 K=32 E=1024 R=64", 1500, 128, 32, 1024, 64, False, dict(mask=0.1)),
    ("N=2000 R=E=64 masked", 2000, 256, 6, 64, 64, True, dict(mask=0.2)),
    ("N=2049 odd K=5 bf16 H=520", 2049, 520, 5, 32, 8, False, dict(mask=0.05)),
    ("N=3000 repeats K=12 E=8", 3000, 128, 12, 8, 4, True, dict(repeats=True)),
    ("N=2500 K=16 E=256 R=32", 2500, 256, 16, 256, 32, True, dict(mask=0.1)),
    ("N=1111 R=64 E=512", 1111, 128, 8, 512, 64, True, dict(mask=0.05)),
    ("N=600 K=1", 600, 256, 1, 32, 8, True, {}),
    ("N=300 all masked", 300, 256, 4, 16, 4, True, dict(mask=1.0)),
    ("K=32 E=1024 R=64", 150, 128, 32, 1024, 64, False, dict(mask=0.1)),
    ("repeats K=12 E=8", 200, 128, 12, 8, 4, True, dict(repeats=True)),
    ("H=9216: more chunks than waves", 60, 9216, 8, 64, 8, True, {}),
    ("H=16384 bf16", 33, 16384, 4, 32, 4, False, {}),
]


@pytest.mark.parametrize("name,N,H,K,E,R,fp8,extra", EDGE, ids=[e[0] for e in EDGE])
def test_fused_edge_shapes(o, name, N, H, K, E, R, fp8, extra):
    x, idx = _random(N, H, K, E, R, seed=N + K, **extra)
    S = N * K if extra.get("repeats") else max(N, 1)
    shape = ep.make_shape(N, H, K, E, R, max(N, 1), S, fp8)
    check_fused(o, shape, x, idx, name)


@pytest.mark.parametrize("N", [200, 600])
def test_fused_capacity_overflow_and_bad_ids(o, N):
    """Entries past the capacity are skipped and reported; ids outside
    [-1, E) are masked and reported; both as the separate calls do (one
    launch at 200 tokens, the count-kernel form at 600)."""
    H, K, E, R = 256, 12, 8, 4
    x, idx = _random(N, H, K, E, R, seed=9, repeats=True)
    check_fused(o, ep.make_shape(N, H, K, E, R, N, N, True), x, idx, "capacity overflow")
    rng = np.random.default_rng(5)
    n = N - 20
    x, idx = _random(n, 256, 4, 32, 4, seed=5)
    pos = rng.permutation(idx.size)[:41]
    idx.reshape(-1)[pos] = rng.choice([-7, -2, 32, 132, 1 << 40], size=41)
    check_fused(o, ep.make_shape(n, 256, 4, 32, 4, n, n, True), x, idx, "bad ids")


@pytest.mark.parametrize("N", [150, 700, 1100])
def test_fused_both_status_bits_in_one_call(o, N):
    """Bad ids and entries past the capacity in the same call: both status
    bits are set, by blocks that may run on different XCDs (one launch at
    150 tokens, the count-kernel form at 700, the large-batch form at
    1,100)."""
    H, K, E, R = 256, 12, 8, 4
    x, idx = _random(N, H, K, E, R, seed=N, repeats=True)
    rng = np.random.default_rng(N + 1)
    pos = rng.permutation(idx.size)[:23]
    idx.reshape(-1)[pos] = rng.choice([-9, E, E + 7, 1 << 33], size=23)
    bits = check_fused(o, ep.make_shape(N, H, K, E, R, N, N, True), x, idx, "bad ids and overflow")
    assert bits & ep.EP_STATUS_BAD_EXPERT_ID and bits & ep.EP_STATUS_BAD_SLOT, bits


@pytest.mark.parametrize("N", [100, 400, 1500])
def test_fused_ids_on_an_8_byte_boundary(o, N):
    """topk_idx at a base that is 8- but not 16-byte aligned: the kernel
    reads ids one at a time instead of two per load."""
    x, idx = _random(N, 256, 8, 64, 8, seed=3)
    check_fused(o, ep.make_shape(N, 256, 8, 64, 8, N, N, True), x, idx, "ids at +8 bytes",
                topk_offset=1)


@pytest.mark.parametrize("N", [120, 500, 2000])
def test_fused_matches_separate_calls_and_expand_offsets(o, N):
    """With an expert alignment, expert_offset follows it exactly as ep_layout's
    (the totals block counts every token at 120 tokens, sums the count
    kernel's histograms at 500)."""
    x, idx = _random(N, 256, 8, 64, 8, seed=21, mask=0.1)
    shape = ep.make_shape(N, 256, 8, 64, 8, N, N, True, expert_alignment=128)
    check_fused(o, shape, x, idx, "expert alignment 128")


@pytest.mark.parametrize("fmt", [ep.EP_SCALE_FP32, ep.EP_SCALE_POW2, ep.EP_SCALE_UE8M0],
                         ids=["fp32", "pow2", "ue8m0"])
def test_fused_prefill_full_size(o, fmt):
    """The prefill workload at full size (4,096 tokens x 7,168, group-limited
    top-8 of 256 experts over 8 ranks): the large-batch form, every output
    bit-exact."""
    w = W.WORKLOADS[3]
    inp = W.make_inputs(w)
    check_fused(o, ep.shape_of(w, fmt), inp["x_bits"], inp["topk_idx"], f"full {w.name}")


def test_fused_large_full_size(o):
    """The large workload at full size (16,384 tokens x 7,168 BF16, top-6 of
    256 experts over 8 ranks, a 60 GB receive buffer): 64 ranking blocks, and
    a pack whose last tokens add 63 earlier blocks' counts; every output
    bit-exact."""
    w = W.WORKLOADS[4]
    inp = W.make_inputs(w)
    check_fused(o, ep.shape_of(w), inp["x_bits"], inp["topk_idx"], f"full {w.name}")


def test_fused_skewed_full_size(o):
    """The skewed workload at full size (4,096 tokens x 4,096, Zipf top-6 of 64
    experts over 64 ranks, 10 % masked): one rank per expert, every output
    bit-exact."""
    w = W.WORKLOADS[5]
    inp = W.make_inputs(w)
    check_fused(o, ep.shape_of(w), inp["x_bits"], inp["topk_idx"], f"full {w.name}")



def test_fused_one_workspace_call_after_call(o):
    """One workspace, poisoned once and never cleared, serves an ep_layout
    call (its histogram rows), then ep_layout_dispatch at 3,000, 1,500 and
    3,000 tokens with new routings (local ranks, histogram rows and the pack
    that reads them), the last two enqueued back to back with no wait
    between: no call depends on what an earlier one left in the workspace.
    Every call is bit-exact and its status clean."""
    H, K, E, R = 512, 8, 64, 8
    big = ep.make_shape(3000, H, K, E, R, 3000, 3000, True)
    need = ep.ep_query_sizes(big)["layout_workspace"]
    ws = torch.full((-(-need // 4),), POISON_I32, dtype=torch.int32, device="cuda")
    x, idx = _random(3000, H, K, E, R, seed=41)
    lay_out = {k: torch.empty(n, dtype=dt, device="cuda") for k, n, dt in (
        ("num_tokens_per_rank", R, torch.int32), ("num_tokens_per_expert", E, torch.int32),
        ("is_token_in_rank", 3000 * R, torch.uint8), ("expert_slot", 3000 * K, torch.int32),
        ("rank_slot", 3000 * R, torch.int32), ("expert_offset", E + 1, torch.int32))}
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("ep_layout N=3000 into the shared workspace")
    ep.ep_layout(big, dev(idx), lay_out["num_tokens_per_rank"], lay_out["num_tokens_per_expert"],
                 lay_out["is_token_in_rank"].view(3000, R), lay_out["expert_slot"].view(3000, K),
                 lay_out["rank_slot"].view(3000, R), lay_out["expert_offset"], ws, st)
    torch.cuda.synchronize()
    assert np.array_equal(host(lay_out["expert_slot"]).reshape(3000, K),
                          o.layout(idx, E, R)["expert_slot"])
    check_fused(o, big, x, idx, "first call on the shared workspace", workspace=ws)
    n = 1500
    x2, idx2 = _random(n, H, K, E, R, seed=42, mask=0.05)
    check_fused(o, ep.make_shape(n, H, K, E, R, n, n, True), x2, idx2,
                "smaller call on the shared workspace", workspace=ws)
    x3, idx3 = _random(3000, H, K, E, R, seed=43)
    x4, idx4 = _random(3000, H, K, E, R, seed=44, mask=0.1)
    say("two calls enqueued back to back on the shared workspace")
    r3 = launch_fused(big, x3, idx3, workspace=ws)
    r4 = launch_fused(big, x4, idx4, workspace=ws)
    torch.cuda.synchronize()
    check_fused(o, big, x3, idx3, "back to back, first", result=r3)
    check_fused(o, big, x4, idx4, "back to back, second", result=r4)
