"""The C ABI's host side, without a GPU: the library loads, exports every
function declared in include/*.h, sizes buffers, and rejects bad arguments
before anything is enqueued.

Every call below that passes stand-in pointers is built to fail a host check
(shape, capacity, null, alignment or workspace) that the library runs before
any HIP call, so no kernel is ever launched from here."""
import ctypes
import glob
import os
import re

import pytest

from combine_ep_layout_02_amd import ep
from combine_ep_layout_02_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(ep_\w+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert set(names) >= {"ep_query_sizes", "ep_layout", "ep_dispatch", "ep_combine", "ep_strerror"}
    lib = ep.lib()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"
    assert set(names) == set(ep.EXPORTED)


def test_struct_layout_matches_header():
    text = open(os.path.join(ROOT, "include", "ep.h")).read()
    shape_body = re.search(r"typedef struct \{(.*?)\} ep_shape;", text, re.S).group(1)
    fields = re.findall(r"int32_t\s+(\w+);", shape_body)
    assert tuple(fields) == ep.SHAPE_FIELDS
    sizes_body = re.search(r"typedef struct \{(.*?)\} ep_sizes;", text, re.S).group(1)
    assert tuple(re.findall(r"size_t\s+(\w+);", sizes_body)) == ep.SIZE_FIELDS


def test_strerror_names_every_code():
    for code in range(0, 9):
        assert ep.ep_strerror(code).startswith("EP_")
    assert "unknown" in ep.ep_strerror(99)


@pytest.mark.parametrize("wid", sorted(W.WORKLOADS))
def test_query_sizes_match_the_receive_geometry(wid):
    w = W.WORKLOADS[wid]
    sz = ep.ep_query_sizes(ep.shape_of(w))
    N, H, K, E, R, S = w.num_tokens, w.hidden, w.num_topk, w.num_experts, w.num_ranks, w.expert_capacity
    assert sz["recv_x"] == E * S * H * (1 if w.use_fp8 else 2)
    assert sz["recv_scales"] == (E * S * (H // 128) * 4 if w.use_fp8 else 0)
    assert sz["recv_src_idx"] == E * S * 4
    assert sz["combined_x"] == N * H * 2
    assert sz["is_token_in_rank"] == N * R and sz["rank_slot"] == N * R * 4
    assert sz["expert_slot"] == N * K * 4 and sz["expert_offset"] == (E + 1) * 4
    # ep_layout's histogram rows, one per 256 tokens; above 1,024 tokens
    # ep_layout_dispatch also keeps local slots and local rank slots [N, K]
    blocks = -(-N // 256)
    stride = -(-(E + R) // 4) * 4
    rows = blocks * stride * 4 if blocks > 1 else 0
    assert sz["layout_workspace"] == (rows if N <= 1024 else rows + 2 * N * K * 4)


@pytest.mark.parametrize("hidden", [128, 512, 640, 7168])
def test_scale_buffer_sizes_per_format(hidden):
    """DeepEP V1 Legacy guide §6.3: fp32 scales are one float per 128-channel
    block; UE8M0 scales pack four block exponents per 32-bit word."""
    w = W.WORKLOADS[3].scaled(64, hidden)
    E, S, G = w.num_experts, w.expert_capacity, hidden // 128
    for fmt, want in ((ep.EP_SCALE_FP32, E * S * G * 4), (ep.EP_SCALE_POW2, E * S * G * 4),
                      (ep.EP_SCALE_UE8M0, E * S * ((G + 3) // 4) * 4)):
        sz = ep.ep_query_sizes(ep.shape_of(w, fmt))
        assert sz["recv_scales"] == want
        assert sz["recv_x"] == E * S * hidden


def test_decode_receive_buffer_is_the_pages_shape():
    """Lesson 14 §3 / DeepEP V1 Legacy guide §6.3: each of the 8 ranks
    receives [32, 8 * 128, 7168] FP8 bytes; here the 8 ranks are slices of
    one [256, 1024, 7168] buffer."""
    w = W.WORKLOADS[2]
    sz = ep.ep_query_sizes(ep.shape_of(w))
    assert sz["recv_x"] == 8 * (32 * 8 * 128 * 7168)
    assert sz["recv_scales"] == 8 * (32 * 8 * 128 * (7168 // 128) * 4)


BAD = ctypes.c_void_p(0x1001)   # misaligned stand-in pointer, never dereferenced
OK16 = ctypes.c_void_p(0x1000)  # aligned stand-in pointer, never dereferenced


def _shape(**kw):
    base = dict(num_tokens=300, hidden=256, num_topk=4, num_experts=16, num_ranks=4,
                num_max_dispatch_tokens_per_rank=300, expert_capacity=300, use_fp8=0,
                scale_format=0, expert_alignment=0)
    base.update(kw)
    return ep.ep_shape(*[int(base[f]) for f in ep.SHAPE_FIELDS])


@pytest.mark.parametrize("kw,code", [
    (dict(num_tokens=-1), ep.EP_ERR_SHAPE),
    (dict(hidden=100), ep.EP_ERR_SHAPE),
    (dict(hidden=0), ep.EP_ERR_SHAPE),
    (dict(num_topk=0), ep.EP_ERR_SHAPE),
    (dict(num_experts=15), ep.EP_ERR_SHAPE),       # E % R != 0
    (dict(num_ranks=0), ep.EP_ERR_SHAPE),
    (dict(use_fp8=1, hidden=200), ep.EP_ERR_SHAPE),  # FP8 needs H % 128 == 0
    (dict(use_fp8=2), ep.EP_ERR_SHAPE),
    (dict(scale_format=1), ep.EP_ERR_SHAPE),                 # scale formats are FP8-only
    (dict(use_fp8=1, scale_format=3), ep.EP_ERR_SHAPE),
    (dict(use_fp8=1, scale_format=-1), ep.EP_ERR_SHAPE),
    (dict(expert_alignment=-1), ep.EP_ERR_SHAPE),
    (dict(expert_alignment=ep.EP_MAX_ALIGNMENT + 1), ep.EP_ERR_UNSUPPORTED),
    (dict(num_topk=33), ep.EP_ERR_UNSUPPORTED),
    (dict(num_experts=2048, num_ranks=4), ep.EP_ERR_UNSUPPORTED),
    (dict(num_experts=128, num_ranks=128), ep.EP_ERR_UNSUPPORTED),
    (dict(num_max_dispatch_tokens_per_rank=299), ep.EP_ERR_CAPACITY),  # N > M
    (dict(expert_capacity=299), ep.EP_ERR_CAPACITY),                   # S < M
    (dict(num_tokens=0, num_max_dispatch_tokens_per_rank=0, expert_capacity=0), ep.EP_ERR_CAPACITY),
])
def test_static_shape_errors_are_reported_before_any_launch(kw, code):
    s = _shape(**kw)
    lib = ep.lib()
    out = ep.ep_sizes()
    assert lib.ep_query_sizes(ctypes.byref(s), ctypes.byref(out)) == code
    args9 = [OK16] * 8
    assert lib.ep_layout(ctypes.byref(s), *args9[:7], OK16, ctypes.c_size_t(1 << 30), None, None) == code
    assert lib.ep_dispatch(ctypes.byref(s), *[OK16] * 6, None, None) == code
    assert lib.ep_combine(ctypes.byref(s), *[OK16] * 6, None, None) == code
    assert lib.ep_dispatch_expand(ctypes.byref(s), *[OK16] * 8, None, None) == code
    assert lib.ep_combine_expand(ctypes.byref(s), *[OK16] * 7, None, None) == code
    assert lib.ep_dispatch_normal(ctypes.byref(s), *[OK16] * 9, None, None) == code
    assert lib.ep_combine_normal(ctypes.byref(s), *[OK16] * 6, None, None) == code
    assert _layout_dispatch(lib, s, [OK16] * 13) == code


def _layout_dispatch(lib, s, p, ws_bytes=1 << 30):
    """ep_layout_dispatch with pointer list p = topk_idx, x, ntpr, ntpe,
    is_token_in_rank, expert_slot, rank_slot, expert_offset, workspace,
    recv_x, recv_scales, recv_src_idx, status."""
    return lib.ep_layout_dispatch(ctypes.byref(s), *p[:9], ctypes.c_size_t(ws_bytes), *p[9:], None)


def test_layout_dispatch_argument_checks():
    lib = ep.lib()
    s = _shape()                               # 300 tokens: the two-launch path
    small = _shape(num_tokens=200)             # one launch
    for shape in (s, small):
        for i in (0, 1, 2, 3, 4, 5, 6, 9, 11):  # every pointer but expert_offset, workspace, scales, status
            q = [OK16] * 13
            q[i] = None
            assert _layout_dispatch(lib, shape, q) == ep.EP_ERR_NULL, i
        for i in (0, 1, 2, 3, 5, 6, 7, 9, 10, 11, 12):  # is_token_in_rank is bytes
            q = [OK16] * 13
            q[i] = BAD
            assert _layout_dispatch(lib, shape, q) == ep.EP_ERR_ALIGN, i
        q = [OK16] * 13
        q[1] = ctypes.c_void_p(0x1008)         # x rows need 16 bytes
        assert _layout_dispatch(lib, shape, q) == ep.EP_ERR_ALIGN
    sf = _shape(use_fp8=1)
    q = [OK16] * 13
    q[10] = None                               # FP8 needs the scales
    assert _layout_dispatch(lib, sf, q) == ep.EP_ERR_NULL
    # the workspace is the layout's, needed only above 256 tokens
    need = ep.ep_query_sizes(s)["layout_workspace"]
    assert need > 0
    q = [OK16] * 13
    q[8] = None
    assert _layout_dispatch(lib, s, q, need) == ep.EP_ERR_WORKSPACE
    assert _layout_dispatch(lib, s, [OK16] * 13, need - 1) == ep.EP_ERR_WORKSPACE


def test_null_pointers_are_rejected():
    s = _shape()
    lib = ep.lib()
    assert lib.ep_query_sizes(None, ctypes.byref(ep.ep_sizes())) == ep.EP_ERR_NULL
    assert lib.ep_query_sizes(ctypes.byref(s), None) == ep.EP_ERR_NULL
    p = [OK16] * 7
    for i in range(6):  # topk_idx .. rank_slot (expert_offset is nullable)
        q = list(p)
        q[i] = None
        assert lib.ep_layout(ctypes.byref(s), *q, OK16, ctypes.c_size_t(1 << 30), None, None) == ep.EP_ERR_NULL
    for i in (0, 1, 2, 3, 5):  # x, topk_idx, expert_slot, recv_x, recv_src_idx
        q = [OK16] * 6
        q[i] = None
        assert lib.ep_dispatch(ctypes.byref(s), *q, None, None) == ep.EP_ERR_NULL
    sf = _shape(use_fp8=1)
    assert lib.ep_dispatch(ctypes.byref(sf), OK16, OK16, OK16, OK16, None, OK16, None, None) == ep.EP_ERR_NULL
    for i in (0, 1, 2, 3, 5):  # expert_out, topk_idx, topk_weights, expert_slot, (bias), out
        q = [OK16] * 6
        q[i] = None
        assert lib.ep_combine(ctypes.byref(s), *q, None, None) == ep.EP_ERR_NULL


def test_null_pointers_are_rejected_by_the_other_layouts():
    s = _shape()
    sf = _shape(use_fp8=1, hidden=256)
    lib = ep.lib()
    # expand: x, topk_idx, expert_slot, expert_offset, counts, recv_x, (scales), recv_src_idx
    for i in (0, 1, 2, 3, 4, 5, 7):
        q = [OK16] * 8
        q[i] = None
        assert lib.ep_dispatch_expand(ctypes.byref(s), *q, None, None) == ep.EP_ERR_NULL
    q = [OK16] * 8
    q[6] = None
    assert lib.ep_dispatch_expand(ctypes.byref(sf), *q, None, None) == ep.EP_ERR_NULL
    for i in (0, 1, 2, 3, 4, 6):  # expert_out .. expert_offset, (bias), out
        q = [OK16] * 7
        q[i] = None
        assert lib.ep_combine_expand(ctypes.byref(s), *q, None, None) == ep.EP_ERR_NULL
    # normal: x, topk_idx, (weights), rank_slot, recv_x, (scales), recv_topk_idx, (w), src
    for i in (0, 1, 3, 4, 6, 8):
        q = [OK16] * 9
        q[i] = None
        assert lib.ep_dispatch_normal(ctypes.byref(s), *q, None, None) == ep.EP_ERR_NULL
    q = [OK16] * 9
    q[5] = None
    assert lib.ep_dispatch_normal(ctypes.byref(sf), *q, None, None) == ep.EP_ERR_NULL
    for i in (0, 1, 4, 5):  # x, rank_slot, (w), (bias), combined_x, combined weights given w
        q = [OK16] * 6
        q[i] = None
        assert lib.ep_combine_normal(ctypes.byref(s), *q, None, None) == ep.EP_ERR_NULL


def test_misaligned_pointers_are_rejected_by_the_other_layouts():
    s = _shape(use_fp8=1, hidden=256)
    lib = ep.lib()
    for n, fn in ((8, lib.ep_dispatch_expand), (7, lib.ep_combine_expand),
                  (9, lib.ep_dispatch_normal), (6, lib.ep_combine_normal)):
        for i in range(n):
            q = [OK16] * n
            q[i] = BAD
            assert fn(ctypes.byref(s), *q, None, None) == ep.EP_ERR_ALIGN, (fn.__name__, i)
    # token rows need 16 bytes
    assert lib.ep_dispatch_expand(ctypes.byref(s), ctypes.c_void_p(0x1008), *[OK16] * 7, None,
                                  None) == ep.EP_ERR_ALIGN
    assert lib.ep_combine_normal(ctypes.byref(s), ctypes.c_void_p(0x1008), *[OK16] * 5, None,
                                 None) == ep.EP_ERR_ALIGN
    # the bias row is a token row: 16 bytes
    q = [OK16] * 6
    q[3] = ctypes.c_void_p(0x1008)
    assert lib.ep_combine_normal(ctypes.byref(s), *q, None, None) == ep.EP_ERR_ALIGN
    # recv_topk_idx is int64
    q = [OK16] * 9
    q[6] = ctypes.c_void_p(0x1004)
    assert lib.ep_dispatch_normal(ctypes.byref(s), *q, None, None) == ep.EP_ERR_ALIGN


@pytest.mark.parametrize("wid", sorted(W.WORKLOADS))
@pytest.mark.parametrize("align", [0, 1, 128])
def test_query_sizes_of_the_other_layouts(wid, align):
    """Normal mode: M rows per rank (V1 guide §5.1); expand layout: M*K rows
    plus at most A-1 padding rows per expert (Ascend deep dive, phase 1)."""
    w = W.WORKLOADS[wid]
    sz = ep.ep_query_sizes(ep.shape_of(w, expert_alignment=align))
    N, H, K, E, R, M = (w.num_tokens, w.hidden, w.num_topk, w.num_experts, w.num_ranks,
                        w.num_max_dispatch_tokens_per_rank)
    b = 1 if w.use_fp8 else 2
    g = H // 128 if w.use_fp8 else 0
    assert sz["recv_x_normal"] == R * M * H * b and sz["recv_scales_normal"] == R * M * g * 4
    assert sz["recv_topk_idx"] == R * M * K * 8 and sz["recv_topk_weights"] == R * M * K * 4
    assert sz["recv_src_idx_normal"] == R * M * 4 and sz["expert_out_normal"] == R * M * H * 2
    assert sz["combined_topk_weights"] == N * K * 4
    T = M * K + E * (max(align, 1) - 1)
    assert T == ep.expand_rows(ep.shape_of(w, expert_alignment=align))
    assert sz["recv_x_expand"] == T * H * b and sz["recv_scales_expand"] == T * g * 4
    assert sz["recv_src_idx_expand"] == T * 4 and sz["expert_out_expand"] == T * H * 2


def test_misaligned_pointers_are_rejected():
    s = _shape()
    lib = ep.lib()
    for i in (0, 1, 2, 4, 5, 6):  # is_token_in_rank (3) is bytes: any address is aligned
        q = [OK16] * 7
        q[i] = BAD
        assert lib.ep_layout(ctypes.byref(s), *q, OK16, ctypes.c_size_t(1 << 30), None, None) == ep.EP_ERR_ALIGN
    assert lib.ep_layout(ctypes.byref(s), *[OK16] * 7, ctypes.c_void_p(0x1008),
                         ctypes.c_size_t(1 << 30), None, None) == ep.EP_ERR_ALIGN  # workspace needs 16 B
    for i in range(6):
        q = [OK16] * 6
        q[i] = BAD
        assert lib.ep_dispatch(ctypes.byref(s), *q, None, None) == ep.EP_ERR_ALIGN
    assert lib.ep_dispatch(ctypes.byref(s), ctypes.c_void_p(0x1008), *[OK16] * 5, None, None) == ep.EP_ERR_ALIGN
    for i in range(6):
        q = [OK16] * 6
        q[i] = BAD
        assert lib.ep_combine(ctypes.byref(s), *q, None, None) == ep.EP_ERR_ALIGN
    for i in (4, 5):  # bias and combined_x are token rows: 16 bytes
        q = [OK16] * 6
        q[i] = ctypes.c_void_p(0x1008)
        assert lib.ep_combine(ctypes.byref(s), *q, None, None) == ep.EP_ERR_ALIGN


def test_layout_workspace_is_checked():
    s = _shape(num_tokens=1000, num_max_dispatch_tokens_per_rank=1000, expert_capacity=1000)
    need = ep.ep_query_sizes(s)["layout_workspace"]
    assert need > 0
    lib = ep.lib()
    assert lib.ep_layout(ctypes.byref(s), *[OK16] * 7, None, ctypes.c_size_t(need), None, None) == ep.EP_ERR_WORKSPACE
    assert lib.ep_layout(ctypes.byref(s), *[OK16] * 7, OK16, ctypes.c_size_t(need - 1), None, None) == ep.EP_ERR_WORKSPACE


def test_layout_noalloc_static_errors():
    """ep_layout_noalloc: a shape whose histograms exceed the static scratch,
    a bad shape, null and misaligned pointers are refused on the host, before
    the device's scratch address is looked up."""
    lib = ep.lib()
    big = _shape(num_tokens=300_000, num_topk=8, num_experts=256, num_ranks=8,
                 num_max_dispatch_tokens_per_rank=300_000,
                 expert_capacity=300_000)
    assert ep.ep_query_sizes(big)["layout_workspace"] > ep.EP_NOALLOC_SCRATCH_BYTES
    call = lambda sh, *p: lib.ep_layout_noalloc(ctypes.byref(sh), *p, None, None)
    assert call(big, *[OK16] * 7) == ep.EP_ERR_SCRATCH
    assert call(_shape(num_ranks=3), *[OK16] * 7) == ep.EP_ERR_SHAPE
    assert call(_shape(), OK16, None, *[OK16] * 5) == ep.EP_ERR_NULL
    assert call(_shape(), BAD, *[OK16] * 6) == ep.EP_ERR_ALIGN


def test_probe_argument_checks():
    lib = ep.lib()
    assert lib.ep_probe_e4m3fn(OK16, OK16, OK16, ctypes.c_int64(6), None) == ep.EP_ERR_SHAPE
    assert lib.ep_probe_e4m3fn(None, OK16, OK16, ctypes.c_int64(8), None) == ep.EP_ERR_NULL
    assert lib.ep_probe_e4m3fn(OK16, None, None, ctypes.c_int64(8), None) == ep.EP_ERR_NULL
    assert lib.ep_probe_e4m3fn(BAD, OK16, OK16, ctypes.c_int64(8), None) == ep.EP_ERR_ALIGN
    assert lib.ep_probe_e4m3fn(OK16, OK16, OK16, ctypes.c_int64(0), None) == ep.EP_OK


def test_binding_refuses_cpu_tensors():
    import torch

    s = _shape()
    with pytest.raises(ValueError):
        ep.ep_combine(s, torch.zeros(4, dtype=torch.int16), torch.zeros(4, dtype=torch.int64),
                      torch.zeros(4), torch.zeros(4, dtype=torch.int32),
                      torch.zeros(4, dtype=torch.int16), stream=0)


def test_gating_argument_checks():
    """ep_group_limited_topk: group rules are checked before any launch."""
    s = _shape(num_experts=16, num_ranks=4, num_topk=4)
    lib = ep.lib()
    call = lambda sh, G, TG, *p, rule=0: lib.ep_group_limited_topk(ctypes.byref(sh), G, TG, rule,
                                                                       *p, None)
    for G, TG, code in ((5, 2, ep.EP_ERR_SHAPE), (0, 1, ep.EP_ERR_SHAPE), (4, 0, ep.EP_ERR_SHAPE),
                        (4, 5, ep.EP_ERR_SHAPE), (8, 1, ep.EP_ERR_SHAPE),  # K=4 > 1 * 16/8
                        (128, 1, ep.EP_ERR_UNSUPPORTED)):
        assert call(s, G, TG, OK16, OK16, OK16) == code, (G, TG)
    assert call(s, 4, 2, None, OK16, OK16) == ep.EP_ERR_NULL
    assert call(s, 4, 2, OK16, None, OK16) == ep.EP_ERR_NULL
    assert call(s, 4, 2, BAD, OK16, OK16) == ep.EP_ERR_ALIGN
    assert call(s, 4, 2, OK16, ctypes.c_void_p(0x1004), OK16) == ep.EP_ERR_ALIGN
    assert call(s, 4, 2, OK16, OK16, BAD) == ep.EP_ERR_ALIGN
    assert call(_shape(num_tokens=-1), 4, 2, OK16, OK16, OK16) == ep.EP_ERR_SHAPE
    for rule in (-1, 2):
        assert call(s, 4, 2, OK16, OK16, OK16, rule=rule) == ep.EP_ERR_SHAPE
    assert call(s, 4, 2, None, OK16, OK16, rule=ep.EP_GATE_SUM_SIGMOID) == ep.EP_ERR_NULL


def test_combine_helper_checks_expert_out_shape():
    """ep.combine refuses expert outputs whose leading dims are not [E, S]
    before any call into the library."""
    import torch

    s = ep.make_shape(4, 8, 2, 8, 2, 4, 4, False)
    z = lambda *shape, dt=torch.int32: torch.zeros(shape, dtype=dt)
    h = ep.Handle(s, z(4, 2, dt=torch.int64), z(2), z(8), z(4, 2, dt=torch.uint8), z(4, 2), z(4, 2),
                  z(9), z(1))
    with pytest.raises(ValueError):
        ep.combine(torch.zeros((8, 5, 8), dtype=torch.bfloat16), h, torch.zeros((4, 2)))
