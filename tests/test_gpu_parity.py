"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Bar: layout outputs, FP8 bytes, fp32 scales, BF16 rows and recv_src_idx are
bit-exact; the combine is within 1 bf16 ulp or 8e-3 relative of the oracle
(and is expected to be bit-identical, since both sides run the same k-ordered
fp32 FMA chain; that is asserted separately).  Outputs start poisoned, so an
element the kernels fail to write is caught, and receive rows past each
expert's count must still hold the poison afterwards.
"""
import numpy as np
import pytest
import torch

import oracle
import pins
from cases import small_cases
from combine_ep_layout_02_amd import ep
from combine_ep_layout_02_amd import workloads as W
from gpu_helpers import (POISON_SCALE_BITS, POISON_SRC, POISON_X8, POISON_X16, DispatchRun,
                         LayoutRun, dev, gather_rows, host, place_expert_rows, run_combine, say,
                         unwritten_rows_intact, written_rows)

pytestmark = pytest.mark.gpu

LAYOUT_KEYS = ("num_tokens_per_rank", "num_tokens_per_expert", "is_token_in_rank", "expert_slot",
               "rank_slot", "expert_offset")
FORMATS = [ep.EP_SCALE_POW2, ep.EP_SCALE_UE8M0]  # beside the default EP_SCALE_FP32


@pytest.fixture(scope="module")
def o():
    return oracle.get()


def first_diff(a, b):
    d = np.argwhere(np.asarray(a) != np.asarray(b))
    return None if d.size == 0 else (tuple(d[0]), np.asarray(a)[tuple(d[0])], np.asarray(b)[tuple(d[0])])


def oracle_capacity(counts, S):
    """Rows per expert for the oracle's buffers: just enough for the largest
    count (saves host memory), but exactly S when some count exceeds S, so
    both sides drop the same entries past the capacity."""
    top = int(counts.max()) if counts.size else 0
    return S if top > S else max(1, top)


def check_layout(o, shape, topk_idx, name):
    say(f"ep_layout {name} N={shape.num_tokens} K={shape.num_topk} E={shape.num_experts} R={shape.num_ranks}")
    run = LayoutRun(shape, topk_idx)
    got = run.numpy()
    want = o.layout(topk_idx, shape.num_experts, shape.num_ranks)
    for key in LAYOUT_KEYS:
        assert np.array_equal(got[key], want[key]), (name, key, first_diff(got[key], want[key]))
    want_status = want["status"]  # oracle reports the bad-id bit the same way
    assert got["status"] == want_status, (name, got["status"], want_status)
    return run, want


def check_dispatch(o, shape, inp, run, lay, name):
    E, S, H = shape.num_experts, shape.expert_capacity, shape.hidden
    say(f"ep_dispatch {name} fp8={shape.use_fp8} scale_format={shape.scale_format} S={S} H={H}")
    d = DispatchRun(shape, inp["x_bits"], run.topk_idx, run.expert_slot)
    torch.cuda.synchronize()
    counts = lay["num_tokens_per_expert"]
    s_or = oracle_capacity(counts, S)
    rx, rs, src, st = o.pack(inp["x_bits"], inp["topk_idx"], lay["expert_slot"], E, s_or,
                             bool(shape.use_fp8), scale_format=shape.scale_format)
    rows_gpu = written_rows(counts, S)
    rows_or = written_rows(counts, s_or)
    got_x = gather_rows(d.recv_x, rows_gpu)
    want_x = rx.reshape(E * s_or, H)[rows_or]
    assert np.array_equal(got_x, want_x), (name, "recv_x", first_diff(got_x, want_x))
    got_src = gather_rows(d.recv_src_idx, rows_gpu)
    assert np.array_equal(got_src, src.reshape(-1)[rows_or]), (name, "recv_src_idx")
    if shape.use_fp8:
        got_sc = gather_rows(d.recv_scales.view(torch.int32), rows_gpu)
        want_sc = rs.reshape(E * s_or, rs.shape[-1])[rows_or].view(np.int32)
        assert np.array_equal(got_sc, want_sc), (name, "recv_scales", first_diff(got_sc, want_sc))
        assert unwritten_rows_intact(d.recv_x, counts, POISON_X8)
        assert unwritten_rows_intact(d.recv_scales.view(torch.int32), counts, POISON_SCALE_BITS)
    else:
        assert unwritten_rows_intact(d.recv_x, counts, int(POISON_X16))
    assert unwritten_rows_intact(d.recv_src_idx, counts, POISON_SRC)
    status = int(d.status.item()) & 0xFFFFFFFF
    assert status == st, (name, status, st)
    return d, rx, s_or


def check_combine(o, shape, inp, run, lay, y_dev, y_or, s_or, name, weights=None, token_sample=None):
    """Combine on device rows y_dev [E, S, H] against the oracle on y_or
    [E, s_or, H] holding the same rows."""
    E = shape.num_experts
    w = inp["topk_weights"] if weights is None else weights
    say(f"ep_combine {name}")
    got, st = run_combine(shape, y_dev, run.topk_idx, w, run.expert_slot)
    idx, slot = inp["topk_idx"], lay["expert_slot"]
    if token_sample is not None:
        got, idx, slot, w = got[token_sample], idx[token_sample], slot[token_sample], w[token_sample]
    want, st_or = o.combine(y_or, idx, w, slot, E, s_or)
    if token_sample is None:
        assert st == st_or, (name, "combine status", st, st_or)
    pins.assert_combine_close(got, pins.bf16_to_f64(want), f"{name} combine vs oracle")
    ndiff = int((got != want).sum())
    say(f"  combine elements not bit-identical to the oracle: {ndiff} of {got.size}")
    assert ndiff == 0, f"{name}: within tolerance but {ndiff} elements not bit-identical"
    return got


def check_path(o, w, inp, name, scale_format=ep.EP_SCALE_FP32):
    shape = ep.shape_of(w, scale_format)
    run, lay = check_layout(o, shape, inp["topk_idx"], name)
    check_dispatch(o, shape, inp, run, lay, name)
    E, S, H = w.num_experts, w.expert_capacity, w.hidden
    y = place_expert_rows(inp["expert_rows"], inp["topk_idx"], lay["expert_slot"], E, S, H)
    s_or = oracle_capacity(lay["num_tokens_per_expert"], S)
    y_or = pins.place_rows(inp["expert_rows"], inp["topk_idx"], lay["expert_slot"], E, s_or)
    check_combine(o, shape, inp, run, lay, y, y_or, s_or, name)


# ------------------------------------------------------------------ FP8 step

def test_fp8_conversion_exhaustive(o):
    """The pack's clamp + E4M3FN conversion (gfx950 instruction and the
    bitwise formulation) against the oracle's encoder for every binary32 in
    [0, 448], and sign symmetry for every negative counterpart; plus the
    structured probe set (codes, midpoints, subnormals, both signs)."""
    top = 0x43E00000
    step = 1 << 26
    for start in range(0, top + 1, step):
        stop = min(start + step, top + 1)
        say(f"ep_probe_e4m3fn bits [{start:#x}, {stop:#x})")
        n = stop - start
        n4 = -(-n // 4) * 4
        bits = torch.arange(start, start + n4, dtype=torch.int64, device="cuda").clamp_(max=top)
        v = bits.to(torch.int32).view(torch.float32)
        hw = torch.empty(n4, dtype=torch.uint8, device="cuda")
        sw = torch.empty(n4, dtype=torch.uint8, device="cuda")
        ep.ep_probe_e4m3fn(v, hw, sw)
        hw_neg = torch.empty_like(hw)
        ep.ep_probe_e4m3fn(-v, hw_neg, None)
        assert torch.equal(hw, sw), "hardware and bitwise conversions differ"
        assert torch.equal(hw_neg, hw | 0x80), "negative inputs are not sign-symmetric"
        want = o.e4m3fn_encode(v.cpu().numpy())
        got = hw.cpu().numpy()
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, f"conversion differs from the oracle at {v.cpu().numpy()[bad[:4]]}"
    vals = pins.fp8_probe_values()
    vals = np.concatenate([vals, np.zeros((-vals.size) % 4, np.float32)])
    d = dev(vals)
    hw = torch.empty(vals.size, dtype=torch.uint8, device="cuda")
    sw = torch.empty_like(hw)
    ep.ep_probe_e4m3fn(d, hw, sw)
    assert np.array_equal(hw.cpu().numpy(), o.e4m3fn_encode(vals))
    assert np.array_equal(sw.cpu().numpy(), o.e4m3fn_encode(vals))


# -------------------------------------------------------------- the workloads

def test_layout_full_size_all_workloads(o):
    for wid, w in W.WORKLOADS.items():
        inp = W.make_inputs(w.scaled(w.num_tokens, 128))  # routing recipe at full N
        check_layout(o, ep.shape_of(w), inp["topk_idx"], w.name)


@pytest.mark.parametrize("case", range(5))
def test_path_small(o, case):
    w, inp = small_cases()[case]
    check_path(o, w, inp, f"small {w.name} N={w.num_tokens} H={w.hidden}")


@pytest.mark.parametrize("wid", [1, 2, 3, 5])
def test_path_full_size(o, wid):
    w = W.WORKLOADS[wid]
    inp = W.make_inputs(w, with_expert_rows=True)
    check_path(o, w, inp, f"full {w.name}")


@pytest.mark.parametrize("fmt", FORMATS, ids=["pow2", "ue8m0"])
def test_scale_formats_full_size(o, fmt):
    """4,096 x 7,168 FP8 prefill with power-of-two / UE8M0 scales."""
    w = W.WORKLOADS[3]
    inp = W.make_inputs(w, with_expert_rows=True)
    check_path(o, w, inp, f"full {w.name} fmt={fmt}", scale_format=fmt)


def test_path_full_size_large_bf16(o):
    """16,384 x 7,168 BF16, top-6 (the Ascend page's 1.4 GB pass): layout and
    pack bit-exact; the combine with the identity expert (the receive buffer
    itself as expert output) matches the oracle and reproduces x exactly."""
    w = W.WORKLOADS[4]
    inp = W.make_inputs(w)
    shape = ep.shape_of(w)
    run, lay = check_layout(o, shape, inp["topk_idx"], w.name)
    d, rx, s_or = check_dispatch(o, shape, inp, run, lay, w.name)
    rows = int((inp["topk_idx"] >= 0).sum())
    assert rows * w.hidden * 2 == 1_409_286_144
    got = check_combine(o, shape, inp, run, lay, d.recv_x, rx, s_or, w.name + " identity")
    assert np.array_equal(pins.bf16_to_f64(got), pins.bf16_to_f64(inp["x_bits"]))


# ------------------------------------------------------- FP8 scale formats

@pytest.mark.parametrize("fmt", FORMATS, ids=["pow2", "ue8m0"])
@pytest.mark.parametrize("case", [1, 2, 4])  # the FP8 small cases
def test_scale_formats_small(o, case, fmt):
    """DeepEP V1 Legacy guide §6.3 round_scale / use_ue8m0: power-of-two
    scales, as fp32 or as packed 8-bit exponents, bit-exact."""
    w, inp = small_cases()[case]
    assert w.use_fp8
    check_path(o, w, inp, f"small {w.name} fmt={fmt}", scale_format=fmt)


@pytest.mark.parametrize("fmt", FORMATS, ids=["pow2", "ue8m0"])
@pytest.mark.parametrize("H", [128, 384, 640, 1152, 1920])
def test_scale_formats_ragged_words(o, H, fmt):
    """Block counts G = H/128 that leave a partly filled UE8M0 word (G % 4 != 0)
    and chunks whose second half holds no block (H % 1024 <= 512)."""
    _edge(o, f"H={H} fmt={fmt}", N=130, H=H, K=6, E=32, R=8, use_fp8=True, mask=0.05,
          scale_format=fmt)


@pytest.mark.parametrize("fmt", [ep.EP_SCALE_FP32] + FORMATS, ids=["fp32", "pow2", "ue8m0"])
def test_scale_formats_exponent_boundaries(o, fmt):
    """Block maxima at 1.75 * 2^E (the power of two 2^(E-8) is exact: 448
    times it equals the maximum), one bf16 step above and below it, at plain
    powers of two, under the 1e-4 floor, and at the extremes of bf16 range:
    every branch of the exponent rule."""
    rng = np.random.default_rng(7)
    N, H = 96, 1024
    G = H // 128
    x = rng.uniform(-1.0, 1.0, (N, G, 128)).astype(np.float32)
    mant = np.array([1.75, 1.75 + 2 ** -7, 1.75 - 2 ** -7, 1.0, 1.5, 1.9921875], np.float32)
    for t in range(N):
        for g in range(G):
            E2 = int(rng.integers(-30, 120))
            m = mant[(t + g) % mant.size]
            x[t, g] *= np.float32(m * 2.0 ** (E2 - 1))
            x[t, g, int(rng.integers(0, 128))] = np.float32((-1) ** t * m * 2.0 ** E2)
    x[0, 0] = 0.0                   # all-zero block: a' = 1e-4
    x[1, 1] = 3e-5                  # under the floor
    x[2, 2, 5] = 3.3895314e38       # largest finite bf16
    x_bits = W.bf16_bits(x.reshape(N, H))
    _edge(o, f"exponent boundaries fmt={fmt}", N=N, H=H, K=4, E=16, R=4, use_fp8=True,
          scale_format=fmt, x_bits=x_bits)


# ------------------------------------------------------------------ edge cases

def _edge(o, name, N, H, K, E, R, use_fp8, topk_idx=None, M=None, S=None, seed=0, mask=0.0,
          scale_format=ep.EP_SCALE_FP32, x_bits=None):
    rng = np.random.default_rng(seed)
    if topk_idx is None:
        topk_idx = np.argsort(rng.random((N, E)), axis=1)[:, :K].astype(np.int64) if K <= E else \
            rng.integers(0, E, size=(N, K))
        if mask:
            topk_idx[rng.random((N, K)) < mask] = -1
    M = max(N, 1) if M is None else M
    S = M if S is None else S
    w = W.Workload(0, name, N, H, K, E, R, M, S, use_fp8, "uniform")
    x = W.bf16_bits(rng.standard_normal((N, H), dtype=np.float32)) if x_bits is None else x_bits
    wts = rng.random((N, K)).astype(np.float32)
    P = int((topk_idx >= 0).sum())
    rows = W.bf16_bits(rng.standard_normal((P, H), dtype=np.float32))
    inp = {"x_bits": x, "topk_idx": topk_idx, "topk_weights": wts, "expert_rows": rows}
    check_path(o, w, inp, name, scale_format)


EDGE = [
    ("N=0", dict(N=0, H=256, K=4, E=16, R=4, use_fp8=True)),
    ("N=1 K=1", dict(N=1, H=128, K=1, E=8, R=2, use_fp8=True)),
    ("N=1 bf16 H=8", dict(N=1, H=8, K=2, E=4, R=2, use_fp8=False)),
    ("all masked", dict(N=70, H=256, K=3, E=8, R=4, use_fp8=True,
                        topk_idx=-np.ones((70, 3), np.int64))),
    ("R=1", dict(N=300, H=128, K=4, E=16, R=1, use_fp8=True)),
    ("R=E=64", dict(N=300, H=256, K=6, E=64, R=64, use_fp8=True, mask=0.2)),
    ("ragged N=257 bf16 H=520", dict(N=257, H=520, K=5, E=32, R=8, use_fp8=False, mask=0.05)),
    ("N=1000 fp8 H=1152", dict(N=1000, H=1152, K=8, E=256, R=8, use_fp8=True)),
    ("N<M, S=R*M", dict(N=50, H=256, K=8, E=64, R=8, use_fp8=True, M=64, S=512)),
    ("K=32 (128-token blocks)", dict(N=333, H=128, K=32, E=256, R=16, use_fp8=True)),
    ("E=1024", dict(N=600, H=128, K=8, E=1024, R=64, use_fp8=True)),
    ("K=32 E=1024 R=64", dict(N=300, H=128, K=32, E=1024, R=64, use_fp8=False, mask=0.1)),
    ("K>E repeats", dict(N=200, H=128, K=12, E=8, R=4, use_fp8=True, S=200 * 12)),
    # 8 < K <= 16 over several layout blocks (the kernels' 16-entry form)
    ("K=10 N=1500 bf16", dict(N=1500, H=256, K=10, E=64, R=8, use_fp8=False, mask=0.05)),
    ("K=16 N=2100 R=32", dict(N=2100, H=128, K=16, E=256, R=32, use_fp8=True)),
    ("K=12 repeats N=1300", dict(N=1300, H=128, K=12, E=8, R=4, use_fp8=True, S=1300 * 12)),
    # repeated experts push counts past the capacity: those entries are
    # skipped by pack and combine and reported as EP_STATUS_BAD_SLOT
    ("capacity overflow", dict(N=200, H=256, K=12, E=8, R=4, use_fp8=True)),
    ("capacity overflow bf16", dict(N=150, H=64, K=10, E=4, R=2, use_fp8=False)),
]


# layout shapes across the kernels' forms: 2 to 33 blocks of 256 tokens, the
# 16- and 32-entry register forms (K = 16, 17), scalar rank rows (R = 6), 64
# ranks on skewed ids (many lanes of a wave on one expert), repeated experts,
# E = 1024, with a bad id in each, against the oracle
LAYOUT_FORMS = [  # (name, N, K, E, R, mask, repeats, alignment)
    ("32 blocks", 8192, 8, 256, 8, 0.0, False, 0),
    ("33 blocks", 8193, 8, 256, 8, 0.0, False, 0),
    ("K=16", 3000, 16, 256, 32, 0.02, False, 0),
    ("K=17", 3000, 17, 256, 32, 0.02, False, 0),
    ("R=6 (scalar rank rows)", 3001, 3, 12, 6, 0.1, False, 128),
    ("R=64 skewed ids", 4096, 6, 64, 64, 0.1, False, 0),
    ("repeats", 2500, 12, 8, 4, 0.05, True, 0),
    ("E=1024 R=64", 1500, 8, 1024, 64, 0.0, False, 32),
    ("2 blocks", 257, 8, 256, 8, 0.0, False, 0),
]


@pytest.mark.parametrize("name,N,K,E,R,mask,repeats,A", LAYOUT_FORMS, ids=[f[0] for f in LAYOUT_FORMS])
def test_layout_forms(o, name, N, K, E, R, mask, repeats, A):
    rng = np.random.default_rng(N + K + E + R)
    if repeats:
        idx = rng.integers(0, E, size=(N, K)).astype(np.int64)
    elif name.endswith("skewed ids"):
        p = 1.0 / np.arange(1, E + 1) ** 1.2
        keys = np.log(p / p.sum())[None, :] + rng.gumbel(size=(N, E))
        idx = np.argsort(-keys, axis=1, kind="stable")[:, :K].astype(np.int64)
    else:
        idx = np.argsort(rng.random((N, E)), axis=1)[:, :K].astype(np.int64)
    if mask:
        idx[rng.random((N, K)) < mask] = -1
    idx[5, 0] = E + 3  # a bad id: treated as masked and reported
    S = N * K if repeats else N
    shape = ep.make_shape(N, 128, K, E, R, N, S, False, ep.EP_SCALE_FP32, A)
    say(f"ep_layout {name} N={N} K={K} E={E} R={R} A={A}")
    run = LayoutRun(shape, idx)
    got = run.numpy()
    want = o.layout(idx, E, R, alignment=max(A, 1))
    for key in LAYOUT_KEYS:
        assert np.array_equal(got[key], want[key]), (name, key, first_diff(got[key], want[key]))
    assert got["status"] == want["status"] == ep.EP_STATUS_BAD_EXPERT_ID


@pytest.mark.parametrize("name,kw", EDGE, ids=[e[0] for e in EDGE])
def test_edge_shapes(o, name, kw):
    _edge(o, name, **kw)


def test_duplicate_experts_in_a_token(o):
    rng = np.random.default_rng(4)
    idx = rng.integers(-1, 6, size=(400, 5)).astype(np.int64)
    idx[::3, 1] = idx[::3, 0]  # force repeats
    _edge(o, "duplicates", N=400, H=256, K=5, E=6, R=3, use_fp8=True, topk_idx=idx, S=400 * 5)


def test_bad_expert_ids_are_masked_and_reported(o):
    rng = np.random.default_rng(5)
    E, R, N, K = 32, 4, 500, 4
    idx = np.argsort(rng.random((N, E)), axis=1)[:, :K].astype(np.int64)
    bad = idx.copy()
    pos = rng.permutation(N * K)[:97]
    bad.reshape(-1)[pos] = rng.choice([-7, -2, E, E + 100, 1 << 40], size=97)
    shape = ep.make_shape(N, 256, K, E, R, N, N, True)
    run, lay = check_layout(o, shape, bad, "bad ids")
    assert lay["status"] & ep.EP_STATUS_BAD_EXPERT_ID
    masked = bad.copy()
    masked[(masked < -1) | (masked >= E)] = -1
    run2, lay2 = check_layout(o, shape, masked, "bad ids masked")
    for key in LAYOUT_KEYS:
        assert np.array_equal(run.numpy()[key], run2.numpy()[key])
    x = W.bf16_bits(rng.standard_normal((N, 256), dtype=np.float32))
    inp = {"x_bits": x, "topk_idx": bad}
    check_dispatch(o, shape, inp, run, lay, "bad ids")


def test_rank_down_emulation(o):
    """A logical rank that drops out (DeepEP V1 Legacy guide §6.4, shrink
    mode masks a rank's traffic): every entry routed to rank 3 is rewritten to
    -1 on the host.  Rank 3 then receives nothing, its region stays
    untouched, and the combine sums the surviving experts only."""
    w = W.WORKLOADS[2]
    inp = W.make_inputs(w)
    L = w.num_experts // w.num_ranks
    idx = inp["topk_idx"].copy()
    idx[(idx // L) == 3] = -1
    rng = np.random.default_rng(6)
    inp = dict(inp, topk_idx=idx)
    inp["expert_rows"] = W.bf16_bits(rng.standard_normal((int((idx >= 0).sum()), w.hidden),
                                                         dtype=np.float32))
    shape = ep.shape_of(w)
    run, lay = check_layout(o, shape, idx, "rank 3 down")
    assert lay["num_tokens_per_rank"][3] == 0
    assert np.all(lay["num_tokens_per_expert"][3 * L:4 * L] == 0)
    check_path(o, w, inp, "rank 3 down")


def test_two_runs_are_bit_identical():
    """Determinism: the whole path twice on the prefill workload gives the
    same bytes (slots come from prefix sums, never from atomics)."""
    w = W.WORKLOADS[3]
    inp = W.make_inputs(w)
    shape = ep.shape_of(w)
    g = torch.Generator(device="cuda")
    g.manual_seed(1)
    y = torch.randn((w.num_experts, w.expert_capacity, w.hidden), dtype=torch.bfloat16,
                    device="cuda", generator=g).view(torch.int16)
    outs = []
    for rep in range(2):
        say(f"determinism run {rep}")
        run = LayoutRun(shape, inp["topk_idx"])
        d = DispatchRun(shape, inp["x_bits"], run.topk_idx, run.expert_slot)
        got, _ = run_combine(shape, y, run.topk_idx, inp["topk_weights"], run.expert_slot)
        r = run.numpy()
        outs.append((r, d.recv_x.cpu(), d.recv_scales.cpu(), d.recv_src_idx.cpu(), got))
        del d
        torch.cuda.empty_cache()
    a, b = outs
    for key in LAYOUT_KEYS:
        assert np.array_equal(a[0][key], b[0][key])
    for i in (1, 2, 3):
        assert torch.equal(a[i].view(torch.uint8) if a[i].dtype == torch.float32 else a[i],
                           b[i].view(torch.uint8) if b[i].dtype == torch.float32 else b[i])
    assert np.array_equal(a[4], b[4])


def test_side_stream_and_handle_reuse(o):
    """Work enqueued on a non-default stream; the layout's expert_slot is
    reused as the handle for a second dispatch (DeepEP V1 Legacy guide
    §5.2(4): the cached handle skips the layout while routing is unchanged)."""
    w = W.WORKLOADS[2]
    inp = W.make_inputs(w, with_expert_rows=True)
    shape = ep.shape_of(w)
    lay = o.layout(inp["topk_idx"], w.num_experts, w.num_ranks)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        say("ep_layout on a side stream")
        run = LayoutRun(shape, inp["topk_idx"], stream=s)
        d1 = DispatchRun(shape, inp["x_bits"], run.topk_idx, run.expert_slot, stream=s)
        d2 = DispatchRun(shape, inp["x_bits"], run.topk_idx, run.expert_slot, stream=s)
    s.synchronize()
    for key in LAYOUT_KEYS:
        assert np.array_equal(run.numpy()[key], lay[key])
    assert torch.equal(d1.recv_x, d2.recv_x) and torch.equal(d1.recv_src_idx, d2.recv_src_idx)


@pytest.mark.parametrize("fused,num_tokens,hidden",
                         [(False, 128, 7168), (True, 128, 7168), (True, 600, 1024),
                          (True, 2048, 1024)],
                         ids=["separate", "ep_layout_dispatch", "ep_layout_dispatch-600-tokens",
                              "ep_layout_dispatch-2048-tokens"])
def test_hip_graph_capture_and_replay(o, fused, num_tokens, hidden):
    """The path is capturable (no allocation, no host sync, no memset): one
    capture of layout + dispatch + combine (the first two as separate calls or
    as one ep_layout_dispatch; at 600 tokens that is the layout's count kernel
    and one fused kernel, at 2,048 the local ranking and the prefix-adding
    pack), replayed several times with eager work in between
    and a new routing copied into the captured input, each replay checked
    against an eager run and the oracle."""
    w = W.WORKLOADS[2].scaled(num_tokens, hidden)
    shape = ep.shape_of(w)
    dev = torch.device("cuda")
    buf = ep.allocate(shape, dev)
    y = torch.empty((w.num_experts, w.expert_capacity, w.hidden), dtype=torch.int16, device=dev)
    idx = torch.empty((w.num_tokens, w.num_topk), dtype=torch.int64, device=dev)
    wts = torch.empty((w.num_tokens, w.num_topk), dtype=torch.float32, device=dev)
    x = torch.empty((w.num_tokens, w.hidden), dtype=torch.int16, device=dev)

    def step():
        if fused:
            ep.ep_layout_dispatch(shape, idx, x, buf["num_tokens_per_rank"],
                                  buf["num_tokens_per_expert"], buf["is_token_in_rank"],
                                  buf["expert_slot"], buf["rank_slot"], buf["expert_offset"],
                                  buf["workspace"], buf["recv_x"], buf["recv_scales"],
                                  buf["recv_src_idx"], buf["status"])
        else:
            ep.ep_layout(shape, idx, buf["num_tokens_per_rank"], buf["num_tokens_per_expert"],
                         buf["is_token_in_rank"], buf["expert_slot"], buf["rank_slot"],
                         buf["expert_offset"], buf["workspace"], buf["status"])
            ep.ep_dispatch(shape, x, idx, buf["expert_slot"], buf["recv_x"], buf["recv_scales"],
                           buf["recv_src_idx"], buf["status"])
        ep.ep_combine(shape, y, idx, wts, buf["expert_slot"], buf["combined_x"], buf["status"])

    def load(seed):
        inp = W.make_inputs(w, seed=seed, with_expert_rows=True)
        lay = o.layout(inp["topk_idx"], w.num_experts, w.num_ranks)
        idx.copy_(torch.from_numpy(inp["topk_idx"]))
        wts.copy_(torch.from_numpy(inp["topk_weights"]))
        x.copy_(torch.from_numpy(inp["x_bits"].view(np.int16)))
        y.copy_(place_expert_rows(inp["expert_rows"], inp["topk_idx"], lay["expert_slot"],
                                  w.num_experts, w.expert_capacity, w.hidden))
        return inp, lay

    def snapshot():
        torch.cuda.synchronize()
        cnt = buf["num_tokens_per_expert"].cpu().numpy()
        rows = written_rows(cnt, w.expert_capacity)
        return {"slot": buf["expert_slot"].cpu().numpy(), "cnt": cnt,
                "rank_slot": buf["rank_slot"].cpu().numpy(),
                "recv_x": gather_rows(buf["recv_x"], rows),
                "recv_scales": gather_rows(buf["recv_scales"].view(torch.int32), rows),
                "out": buf["combined_x"].cpu().numpy()}

    load(7)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep, seed in enumerate((11, 11, 12, 13)):
        say(f"graph replay {rep} (routing seed {seed})")
        inp, lay = load(seed)
        torch.cuda.synchronize()
        step()  # eager reference on the same inputs
        eager = snapshot()
        for key in ("num_tokens_per_expert", "expert_slot", "combined_x"):
            buf[key].fill_(-1)  # ordinary eager work between replays
        graph.replay()
        replay = snapshot()
        for key in eager:
            assert np.array_equal(eager[key], replay[key]), (rep, key)
        assert np.array_equal(replay["slot"], lay["expert_slot"])
        assert np.array_equal(replay["cnt"], lay["num_tokens_per_expert"])
    assert int(buf["status"].item()) == 0


def _layout_into(shape, topk_idx_dev, ws, status):
    N, K, E, R = shape.num_tokens, shape.num_topk, shape.num_experts, shape.num_ranks
    out = {
        "num_tokens_per_rank": torch.full((R,), -5, dtype=torch.int32, device="cuda"),
        "num_tokens_per_expert": torch.full((E,), -5, dtype=torch.int32, device="cuda"),
        "is_token_in_rank": torch.full((N, R), 0xEE, dtype=torch.uint8, device="cuda"),
        "expert_slot": torch.full((N, K), -5, dtype=torch.int32, device="cuda"),
        "rank_slot": torch.full((N, R), -5, dtype=torch.int32, device="cuda"),
        "expert_offset": torch.full((E + 1,), -5, dtype=torch.int32, device="cuda"),
    }
    ep.ep_layout(shape, topk_idx_dev, out["num_tokens_per_rank"], out["num_tokens_per_expert"],
                 out["is_token_in_rank"], out["expert_slot"], out["rank_slot"],
                 out["expert_offset"], ws, status)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def test_layout_workspace_reused_across_sizes(o):
    """One workspace, never cleared, serves layout calls of different sizes
    one after another (its contents on entry are irrelevant)."""
    big = W.WORKLOADS[4]  # 16,384 tokens: 64 blocks
    ws_bytes = ep.ep_query_sizes(ep.shape_of(big))["layout_workspace"]
    ws = torch.full((ws_bytes // 4,), 0x7B7B7B7B, dtype=torch.int32, device="cuda")
    for wid, n in ((4, 16384), (3, 4096), (5, 1000), (3, 257), (4, 16384)):
        w = W.WORKLOADS[wid].scaled(n, 128)
        shape = ep.shape_of(w)
        inp = W.make_inputs(w)
        assert ep.ep_query_sizes(shape)["layout_workspace"] <= ws_bytes
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        say(f"ep_layout N={n} into a shared workspace")
        got = _layout_into(shape, dev(inp["topk_idx"]), ws, status)
        want = o.layout(inp["topk_idx"], w.num_experts, w.num_ranks)
        for key in LAYOUT_KEYS:
            assert np.array_equal(got[key], want[key]), (n, key)
        assert int(status.item()) == 0


def test_two_streams_and_two_host_threads(o):
    """Reentrancy: two independent prefill-shaped steps (different routings,
    inputs and buffers) issued on two streams from two host threads at once
    give exactly what each gives when run alone."""
    import threading

    w = W.WORKLOADS[3].scaled(1500, 1024)
    shape = ep.shape_of(w)
    d = torch.device("cuda")
    runs = []
    for seed in (21, 22):
        inp = W.make_inputs(w, seed=seed)
        buf = ep.allocate(shape, d)
        g = torch.Generator(device=d)
        g.manual_seed(seed)
        runs.append({
            "buf": buf,
            "idx": torch.from_numpy(inp["topk_idx"]).to(d),
            "x": torch.from_numpy(inp["x_bits"].view(np.int16)).to(d),
            "wts": torch.from_numpy(inp["topk_weights"]).to(d),
            "y": torch.randn((w.num_experts, w.expert_capacity, w.hidden), dtype=torch.bfloat16,
                             device=d, generator=g).view(torch.int16),
            "stream": torch.cuda.Stream(),
        })

    def step(r):
        b = r["buf"]
        with torch.cuda.stream(r["stream"]):
            for _ in range(3):
                ep.ep_layout(shape, r["idx"], b["num_tokens_per_rank"], b["num_tokens_per_expert"],
                             b["is_token_in_rank"], b["expert_slot"], b["rank_slot"], b["expert_offset"],
                             b["workspace"], b["status"])
                ep.ep_dispatch(shape, r["x"], r["idx"], b["expert_slot"], b["recv_x"], b["recv_scales"],
                               b["recv_src_idx"], b["status"])
                ep.ep_combine(shape, r["y"], r["idx"], r["wts"], b["expert_slot"], b["combined_x"],
                              b["status"])

    keys = ("expert_slot", "rank_slot", "num_tokens_per_expert", "combined_x", "recv_src_idx")

    def snap(r):
        r["stream"].synchronize()
        return {k: r["buf"][k].cpu().numpy().copy() for k in keys}

    alone = []
    for r in runs:
        for k in keys:  # rows past each expert's count are never written
            r["buf"][k].fill_(-1)
        torch.cuda.synchronize()  # the fills (current stream) before the step (its own stream)
        step(r)
        alone.append(snap(r))
        assert int(r["buf"]["status"].item()) == 0
        for k in keys:
            r["buf"][k].fill_(-1)
    torch.cuda.synchronize()
    say("two host threads, two streams")
    threads = [threading.Thread(target=step, args=(r,)) for r in runs]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    for i, r in enumerate(runs):
        got = snap(r)
        for k in keys:
            assert np.array_equal(got[k], alone[i][k]), (i, k)
        assert int(r["buf"]["status"].item()) == 0


@pytest.mark.parametrize("wid", [2, 1])
def test_three_call_api(o, wid):
    """ep.layout / ep.dispatch / ep.combine (outputs allocated by the binding)
    give what the oracle gives, on the decode workload (FP8) and the tiny one
    (BF16)."""
    w = W.WORKLOADS[wid]
    inp = W.make_inputs(w, with_expert_rows=True)
    E, S, H = w.num_experts, w.expert_capacity, w.hidden
    idx = dev(inp["topk_idx"])
    handle = ep.layout(idx, E, w.num_ranks, w.num_max_dispatch_tokens_per_rank, S)
    x = dev(inp["x_bits"]).view(torch.bfloat16)
    recv_x, recv_scales, recv_src = ep.dispatch(x, handle, use_fp8=w.use_fp8)
    torch.cuda.synchronize()
    lay = o.layout(inp["topk_idx"], E, w.num_ranks)
    for key in ("num_tokens_per_rank", "num_tokens_per_expert", "expert_slot", "rank_slot",
                "is_token_in_rank"):
        assert np.array_equal(host(getattr(handle, key)), lay[key]), key
    cnt = lay["num_tokens_per_expert"]
    s_or = oracle_capacity(cnt, S)
    rx, rs, src, st = o.pack(inp["x_bits"], inp["topk_idx"], lay["expert_slot"], E, s_or, w.use_fp8)
    got_x = recv_x.view(torch.uint8 if w.use_fp8 else torch.int16).cpu().numpy()
    got_src = host(recv_src)
    for e in range(E):
        c = int(cnt[e])
        assert np.array_equal(got_x[e, :c].view(rx.dtype), rx[e, :c]), e
        assert np.array_equal(got_src[e, :c], src[e, :c]), e
        if w.use_fp8:
            assert np.array_equal(host(recv_scales[e, :c]).view(np.int32), rs[e, :c].view(np.int32)), e
    y_or = pins.place_rows(inp["expert_rows"], inp["topk_idx"], lay["expert_slot"], E, s_or)
    y = place_expert_rows(inp["expert_rows"], inp["topk_idx"], lay["expert_slot"], E, S, H)
    out = ep.combine(y.view(torch.bfloat16), handle, dev(inp["topk_weights"]))
    torch.cuda.synchronize()
    want, st_c = o.combine(y_or, inp["topk_idx"], inp["topk_weights"], lay["expert_slot"], E, s_or)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert out.dtype == torch.bfloat16 and np.array_equal(got, want)
    assert int(handle.status.item()) == (lay["status"] | st | st_c)


def test_three_call_api_side_stream_with_workspace(o):
    """ep.layout / ep.dispatch / ep.combine on a stream that is not torch's
    current one, at a batch whose layout needs the histogram workspace (700
    tokens: three count blocks).  The binding allocates on that stream, so the
    caching allocator cannot hand a block the launches still use to other
    work; the current stream is kept busy meanwhile to give a misordered
    allocation the chance to show."""
    w = W.WORKLOADS[3].scaled(700, 1024)
    inp = W.make_inputs(w, seed=4242, with_expert_rows=True)
    E, S, H, R = w.num_experts, w.expert_capacity, w.hidden, w.num_ranks
    assert ep.ep_query_sizes(ep.shape_of(w))["layout_workspace"] > 0
    side = torch.cuda.Stream()
    idx = dev(inp["topk_idx"])
    x = dev(inp["x_bits"]).view(torch.bfloat16)
    wts = dev(inp["topk_weights"])
    lay = o.layout(inp["topk_idx"], E, R)
    y = place_expert_rows(inp["expert_rows"], inp["topk_idx"], lay["expert_slot"], E, S, H)
    side.wait_stream(torch.cuda.current_stream())
    busy = torch.empty(1 << 26, dtype=torch.float32, device="cuda")
    for _ in range(3):
        handle = ep.layout(idx, E, R, w.num_max_dispatch_tokens_per_rank, S, stream=side)
        # work on the current stream that allocates and writes while the side
        # stream runs
        for _ in range(4):
            busy.add_(1.0)
            torch.full((1 << 20,), -7, dtype=torch.int32, device="cuda")
        recv_x, recv_scales, recv_src = ep.dispatch(x, handle, use_fp8=True, stream=side)
        out = ep.combine(y.view(torch.bfloat16), handle, wts, stream=side)
        side.synchronize()
        for key in ("num_tokens_per_rank", "num_tokens_per_expert", "expert_slot", "rank_slot",
                    "is_token_in_rank"):
            assert np.array_equal(host(getattr(handle, key)), lay[key]), key
        cnt = lay["num_tokens_per_expert"]
        s_or = oracle_capacity(cnt, S)
        rx, rs, src, st = o.pack(inp["x_bits"], inp["topk_idx"], lay["expert_slot"], E, s_or, True)
        got_x = recv_x.view(torch.uint8).cpu().numpy()
        got_src = host(recv_src)
        got_sc = host(recv_scales).view(np.int32)
        for e in range(E):
            c = int(cnt[e])
            assert np.array_equal(got_x[e, :c], rx[e, :c]), e
            assert np.array_equal(got_src[e, :c], src[e, :c]), e
            assert np.array_equal(got_sc[e, :c], rs[e, :c].view(np.int32)), e
        y_or = pins.place_rows(inp["expert_rows"], inp["topk_idx"], lay["expert_slot"], E, s_or)
        want, st_c = o.combine(y_or, inp["topk_idx"], inp["topk_weights"], lay["expert_slot"], E, s_or)
        assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), want)
        assert int(handle.status.item()) == 0


def test_prepared_calls_match_plain_calls(o):
    """ep.prepare: the decode step issued three times as prepared calls gives
    exactly what the plain binding gives (and the oracle); preparing
    something that launches nothing is refused."""
    w = W.WORKLOADS[2]
    inp = W.make_inputs(w, with_expert_rows=True)
    shape = ep.shape_of(w)
    d = torch.device("cuda")
    idx, x = dev(inp["topk_idx"]), dev(inp["x_bits"])
    wts = dev(inp["topk_weights"])
    lay = o.layout(inp["topk_idx"], w.num_experts, w.num_ranks)
    y = place_expert_rows(inp["expert_rows"], inp["topk_idx"], lay["expert_slot"], w.num_experts,
                          w.expert_capacity, w.hidden)
    outs = []
    for kind in ("plain", "prepared"):
        b = ep.allocate(shape, d)
        for v in b.values():  # the same fill in both, so unwritten rows compare equal
            if v is not None:
                v.view(torch.uint8).fill_(0x5A)
        b["status"].zero_()
        args = {
            "layout": (ep.ep_layout, shape, idx, b["num_tokens_per_rank"], b["num_tokens_per_expert"],
                       b["is_token_in_rank"], b["expert_slot"], b["rank_slot"], b["expert_offset"],
                       b["workspace"], b["status"]),
            "dispatch": (ep.ep_dispatch, shape, x, idx, b["expert_slot"], b["recv_x"], b["recv_scales"],
                         b["recv_src_idx"], b["status"]),
            "combine": (ep.ep_combine, shape, y, idx, wts, b["expert_slot"], b["combined_x"],
                        b["status"]),
        }
        if kind == "plain":
            for fn, *a in args.values():
                fn(*a)
        else:
            calls = [ep.prepare(fn, *a) for fn, *a in args.values()]
            for _ in range(3):
                for c in calls:
                    c()
        torch.cuda.synchronize()
        outs.append({k: host(v.view(torch.uint8) if v.dtype == torch.float32 else v)
                     for k, v in b.items() if v is not None})
    for k in outs[0]:
        assert np.array_equal(outs[0][k], outs[1][k]), k
    assert np.array_equal(outs[1]["expert_slot"], lay["expert_slot"])
    with pytest.raises(ValueError):
        ep.prepare(ep.make_shape, 1, 8, 1, 1, 1, 1, 1, False)
