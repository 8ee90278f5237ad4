"""Thin ctypes binding of libep_mi355x.so (declared in include/ep.h).

Same entry points as the C ABI: ``ep_query_sizes``, ``ep_layout``, ``ep_layout_noalloc``,
``ep_dispatch``, ``ep_layout_dispatch``, ``ep_combine``, ``ep_dispatch_expand``,
``ep_combine_expand``, ``ep_dispatch_normal``, ``ep_combine_normal``,
``ep_group_limited_topk``, ``ep_logfmt_encode``, ``ep_combine_logfmt``,
``ep_strerror`` (plus ``ep_probe_e4m3fn`` and ``ep_probe_log2_bf16`` from
include/ep_probe.h); and ``layout`` / ``dispatch`` / ``combine``, the path in
three calls that allocate their outputs.  Functions take torch tensors that
already live on the GPU, check dtype / device / contiguity, and pass
``data_ptr()`` and the current HIP stream to the library.  Every step of the path runs in the HIP
kernels; this module only marshals arguments and allocates buffers with torch
on request.  There is no fallback: without the built library every call
raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import dataclasses
import os
import threading
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libep_mi355x.so")

EP_OK = 0
EP_ERR_NULL = 1
EP_ERR_SHAPE = 2
EP_ERR_CAPACITY = 3
EP_ERR_ALIGN = 4
EP_ERR_UNSUPPORTED = 5
EP_ERR_HIP = 6
EP_ERR_WORKSPACE = 7
EP_ERR_SCRATCH = 8
EP_NOALLOC_SCRATCH_BYTES = 1 << 20
EP_STATUS_BAD_EXPERT_ID = 1
EP_STATUS_BAD_SLOT = 2

SHAPE_FIELDS = ("num_tokens", "hidden", "num_topk", "num_experts", "num_ranks",
                "num_max_dispatch_tokens_per_rank", "expert_capacity", "use_fp8", "scale_format",
                "expert_alignment")
EP_SCALE_FP32 = 0
EP_SCALE_POW2 = 1
EP_SCALE_UE8M0 = 2
SIZE_FIELDS = ("recv_x", "recv_scales", "recv_src_idx", "expert_out", "combined_x",
               "num_tokens_per_rank", "num_tokens_per_expert", "is_token_in_rank",
               "expert_slot", "rank_slot", "expert_offset", "layout_workspace",
               "recv_x_normal", "recv_scales_normal", "recv_topk_idx", "recv_topk_weights",
               "recv_src_idx_normal", "expert_out_normal", "combined_topk_weights",
               "recv_x_expand", "recv_scales_expand", "recv_src_idx_expand", "expert_out_expand",
               "logfmt_codes", "logfmt_headers")
EXPORTED = ("ep_query_sizes", "ep_layout", "ep_layout_noalloc", "ep_dispatch", "ep_layout_dispatch", "ep_combine",
            "ep_dispatch_expand",
            "ep_combine_expand", "ep_dispatch_normal", "ep_combine_normal",
            "ep_group_limited_topk", "ep_logfmt_encode", "ep_combine_logfmt", "ep_strerror",
            "ep_probe_e4m3fn", "ep_probe_log2_bf16")
EP_MAX_GROUPS = 64
EP_GATE_MAX_SOFTMAX = 0
EP_GATE_SUM_SIGMOID = 1
EP_MAX_ALIGNMENT = 1024


class ep_shape(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int32) for f in SHAPE_FIELDS]


class ep_sizes(ctypes.Structure):
    _fields_ = [(f, ctypes.c_size_t) for f in SIZE_FIELDS]


class EpError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {ep_strerror(code)} (code {code})")


_LIB: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIBRARY):
            raise RuntimeError(f"{LIBRARY} is not built: run `python -m combine_ep_layout_02_amd.build`."
                               " The GPU path has no fallback.")
        L = ctypes.CDLL(LIBRARY)
        vp, sz, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64
        sp = ctypes.POINTER(ep_shape)
        L.ep_query_sizes.argtypes = [sp, ctypes.POINTER(ep_sizes)]
        L.ep_layout.argtypes = [sp] + [vp] * 8 + [sz, vp, vp]
        L.ep_layout_noalloc.argtypes = [sp] + [vp] * 9
        L.ep_dispatch.argtypes = [sp] + [vp] * 8
        L.ep_layout_dispatch.argtypes = [sp] + [vp] * 9 + [sz] + [vp] * 5
        L.ep_combine.argtypes = [sp] + [vp] * 8
        L.ep_dispatch_expand.argtypes = [sp] + [vp] * 10
        L.ep_combine_expand.argtypes = [sp] + [vp] * 9
        L.ep_dispatch_normal.argtypes = [sp] + [vp] * 11
        L.ep_combine_normal.argtypes = [sp] + [vp] * 8
        L.ep_group_limited_topk.argtypes = [sp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32] + [vp] * 4
        L.ep_probe_e4m3fn.argtypes = [vp, vp, vp, i64, vp]
        L.ep_probe_log2_bf16.argtypes = [vp, vp, i64, vp]
        L.ep_logfmt_encode.argtypes = [sp] + [vp] * 7
        L.ep_combine_logfmt.argtypes = [sp] + [vp] * 9
        L.ep_strerror.argtypes = [ctypes.c_int]
        L.ep_strerror.restype = ctypes.c_char_p
        for name in EXPORTED:
            if name != "ep_strerror":
                getattr(L, name).restype = ctypes.c_int
        _LIB = L
    return _LIB


# ---- calls, and calls prepared once for re-issue -----------------------------
_RECORD = threading.local()


def _call(name: str, *args) -> int:
    """Call entry point ``name`` with converted arguments, or, while
    ``prepare`` records, keep the call instead of making it."""
    fn = getattr(lib(), name)
    calls = getattr(_RECORD, "calls", None)
    if calls is not None:
        calls.append((fn, args, name))
        return EP_OK
    return fn(*args)


class Prepared:
    """One call of an entry point whose arguments were checked and converted
    once by ``prepare``: calling it issues the same call again (the same
    pointers and the same stream), without the per-call checks and
    conversions of the binding, for loops that re-issue one step many times.
    The tensors it was prepared with are kept alive here; their storage must
    not be replaced (an in-place resize would leave a stale pointer)."""
    __slots__ = ("_fn", "_args", "_name", "_keep")

    def __init__(self, fn, args, name, keep):
        self._fn, self._args, self._name, self._keep = fn, args, name, keep

    def __call__(self) -> None:
        rc = self._fn(*self._args)
        if rc != EP_OK:
            raise EpError(rc, self._name)


def prepare(entry, *args, **kwargs) -> Prepared:
    """``entry`` (one of this module's ep_* functions) with its arguments,
    checked and converted now, as a ``Prepared`` call.  ``stream`` defaults
    to torch's current stream at preparation time."""
    _RECORD.calls = []
    try:
        entry(*args, **kwargs)
        calls = _RECORD.calls
    finally:
        _RECORD.calls = None
    if len(calls) != 1:
        raise ValueError(f"{getattr(entry, '__name__', entry)} is not a launching entry point")
    fn, cargs, name = calls[0]
    return Prepared(fn, cargs, name, (args, kwargs))


def make_shape(num_tokens: int, hidden: int, num_topk: int, num_experts: int, num_ranks: int,
               num_max_dispatch_tokens_per_rank: int, expert_capacity: int,
               use_fp8: bool, scale_format: int = EP_SCALE_FP32,
               expert_alignment: int = 0) -> ep_shape:
    return ep_shape(int(num_tokens), int(hidden), int(num_topk), int(num_experts), int(num_ranks),
                    int(num_max_dispatch_tokens_per_rank), int(expert_capacity), int(bool(use_fp8)),
                    int(scale_format), int(expert_alignment))


def shape_of(workload, scale_format: int = EP_SCALE_FP32, expert_alignment: int = 0) -> ep_shape:
    """ep_shape of a ``workloads.Workload`` (FP8 workloads may pick a scale
    format; ``expert_alignment`` sets the expand layout's queue alignment)."""
    w = workload
    return make_shape(w.num_tokens, w.hidden, w.num_topk, w.num_experts, w.num_ranks,
                      w.num_max_dispatch_tokens_per_rank, w.expert_capacity, w.use_fp8,
                      scale_format if w.use_fp8 else EP_SCALE_FP32, expert_alignment)


def expand_rows(shape: ep_shape) -> int:
    """Rows T of the expand-layout buffers: M * K + E * (A - 1)."""
    a = max(int(shape.expert_alignment), 1)
    return shape.num_max_dispatch_tokens_per_rank * shape.num_topk + shape.num_experts * (a - 1)


def scale_row_elems(shape: ep_shape) -> int:
    """Scale elements per receive row: H/128 floats, or ceil(H/512) UE8M0 words."""
    g = shape.hidden // 128
    return (g + 3) // 4 if shape.scale_format == EP_SCALE_UE8M0 else g


def ep_strerror(code: int) -> str:
    return lib().ep_strerror(int(code)).decode()


def ep_query_sizes(shape: ep_shape) -> dict:
    out = ep_sizes()
    rc = lib().ep_query_sizes(ctypes.byref(shape), ctypes.byref(out))
    if rc != EP_OK:
        raise EpError(rc, "ep_query_sizes")
    return {f: int(getattr(out, f)) for f in SIZE_FIELDS}


# torch's current stream as a raw pointer: the private query is about 20x
# cheaper per call than torch.cuda.current_stream(); the public one stands in
# where it is missing.
_RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, ref: torch.Tensor) -> int:
    """The stream argument as an integer handle: ``stream`` (a torch stream
    or a raw handle), else torch's current stream on ``ref``'s device."""
    if stream is None:
        if _RAW_STREAM is not None:
            return _RAW_STREAM(ref.get_device())
        stream = torch.cuda.current_stream(ref.device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: Optional[torch.Tensor], name: str, dtypes, numel: Optional[int] = None):
    """The device address of ``t`` (None for None) after the checks every
    pointer argument gets: a contiguous GPU tensor of an accepted dtype with
    at least ``numel`` elements."""
    if t is None:
        return None
    if (not t.is_cuda or not t.is_contiguous() or t.dtype not in dtypes
            or (numel is not None and t.numel() < numel)):
        _bad_tensor(t, name, dtypes, numel)
    return t.data_ptr()


def _bad_tensor(t: torch.Tensor, name: str, dtypes, numel: Optional[int]):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    raise ValueError(f"{name} has {t.numel()} elements, needs at least {numel}")


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_I64 = (torch.int64,)
_I32 = (torch.int32,)
_U8 = (torch.uint8, torch.bool)
_F32 = (torch.float32,)
_STATUS = (torch.int32, torch.uint32)
_FP8 = (torch.uint8, torch.float8_e4m3fn)


def ep_layout(shape: ep_shape, topk_idx: torch.Tensor, num_tokens_per_rank: torch.Tensor,
              num_tokens_per_expert: torch.Tensor, is_token_in_rank: torch.Tensor,
              expert_slot: torch.Tensor, rank_slot: torch.Tensor,
              expert_offset: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
              status: Optional[torch.Tensor] = None, stream=None) -> None:
    """Dispatch layout; see ``ep_layout`` in include/ep.h."""
    N, K, E, R = shape.num_tokens, shape.num_topk, shape.num_experts, shape.num_ranks
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = _call("ep_layout", 
        ctypes.byref(shape), _ptr(topk_idx, "topk_idx", _I64, N * K),
        _ptr(num_tokens_per_rank, "num_tokens_per_rank", _I32, R),
        _ptr(num_tokens_per_expert, "num_tokens_per_expert", _I32, E),
        _ptr(is_token_in_rank, "is_token_in_rank", _U8, N * R),
        _ptr(expert_slot, "expert_slot", _I32, N * K), _ptr(rank_slot, "rank_slot", _I32, N * R),
        _ptr(expert_offset, "expert_offset", _I32, E + 1),
        _ptr(workspace, "workspace", (torch.uint8, torch.int32)), ctypes.c_size_t(ws_bytes),
        _ptr(status, "status", _STATUS, 1), _stream(stream, num_tokens_per_expert))
    if rc != EP_OK:
        raise EpError(rc, "ep_layout")


def ep_layout_noalloc(shape: ep_shape, topk_idx: torch.Tensor, num_tokens_per_rank: torch.Tensor,
                      num_tokens_per_expert: torch.Tensor, is_token_in_rank: torch.Tensor,
                      expert_slot: torch.Tensor, rank_slot: torch.Tensor,
                      expert_offset: Optional[torch.Tensor] = None,
                      status: Optional[torch.Tensor] = None, stream=None) -> None:
    """Dispatch layout with the library's static per-device scratch instead of
    a workspace; see ``ep_layout_noalloc`` in include/ep.h."""
    N, K, E, R = shape.num_tokens, shape.num_topk, shape.num_experts, shape.num_ranks
    rc = _call("ep_layout_noalloc", 
        ctypes.byref(shape), _ptr(topk_idx, "topk_idx", _I64, N * K),
        _ptr(num_tokens_per_rank, "num_tokens_per_rank", _I32, R),
        _ptr(num_tokens_per_expert, "num_tokens_per_expert", _I32, E),
        _ptr(is_token_in_rank, "is_token_in_rank", _U8, N * R),
        _ptr(expert_slot, "expert_slot", _I32, N * K), _ptr(rank_slot, "rank_slot", _I32, N * R),
        _ptr(expert_offset, "expert_offset", _I32, E + 1),
        _ptr(status, "status", _STATUS, 1), _stream(stream, num_tokens_per_expert))
    if rc != EP_OK:
        raise EpError(rc, "ep_layout_noalloc")


def ep_dispatch(shape: ep_shape, x: torch.Tensor, topk_idx: torch.Tensor, expert_slot: torch.Tensor,
                recv_x: torch.Tensor, recv_scales: Optional[torch.Tensor],
                recv_src_idx: torch.Tensor, status: Optional[torch.Tensor] = None,
                stream=None) -> None:
    """Dispatch pack; see ``ep_dispatch`` in include/ep.h."""
    N, H, K, E, S = shape.num_tokens, shape.hidden, shape.num_topk, shape.num_experts, \
        shape.expert_capacity
    rows = E * S
    rx_types = _FP8 if shape.use_fp8 else _BF16
    rc = _call("ep_dispatch", 
        ctypes.byref(shape), _ptr(x, "x", _BF16, N * H), _ptr(topk_idx, "topk_idx", _I64, N * K),
        _ptr(expert_slot, "expert_slot", _I32, N * K), _ptr(recv_x, "recv_x", rx_types, rows * H),
        (_ptr(recv_scales, "recv_scales", _STATUS, rows * ((H // 128 + 3) // 4))
         if shape.scale_format == EP_SCALE_UE8M0 else
         _ptr(recv_scales, "recv_scales", _F32, rows * (H // 128))) if shape.use_fp8 else None,
        _ptr(recv_src_idx, "recv_src_idx", _I32, rows), _ptr(status, "status", _STATUS, 1),
        _stream(stream, recv_x))
    if rc != EP_OK:
        raise EpError(rc, "ep_dispatch")


def ep_layout_dispatch(shape: ep_shape, topk_idx: torch.Tensor, x: torch.Tensor,
                       num_tokens_per_rank: torch.Tensor, num_tokens_per_expert: torch.Tensor,
                       is_token_in_rank: torch.Tensor, expert_slot: torch.Tensor,
                       rank_slot: torch.Tensor, expert_offset: Optional[torch.Tensor],
                       workspace: Optional[torch.Tensor], recv_x: torch.Tensor,
                       recv_scales: Optional[torch.Tensor], recv_src_idx: torch.Tensor,
                       status: Optional[torch.Tensor] = None, stream=None) -> None:
    """Layout and dispatch pack in one call; see ``ep_layout_dispatch`` in
    include/ep.h."""
    N, H, K, E, R, S = shape.num_tokens, shape.hidden, shape.num_topk, shape.num_experts, \
        shape.num_ranks, shape.expert_capacity
    rows = E * S
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = _call("ep_layout_dispatch", 
        ctypes.byref(shape), _ptr(topk_idx, "topk_idx", _I64, N * K), _ptr(x, "x", _BF16, N * H),
        _ptr(num_tokens_per_rank, "num_tokens_per_rank", _I32, R),
        _ptr(num_tokens_per_expert, "num_tokens_per_expert", _I32, E),
        _ptr(is_token_in_rank, "is_token_in_rank", _U8, N * R),
        _ptr(expert_slot, "expert_slot", _I32, N * K), _ptr(rank_slot, "rank_slot", _I32, N * R),
        _ptr(expert_offset, "expert_offset", _I32, E + 1),
        _ptr(workspace, "workspace", (torch.uint8, torch.int32)), ctypes.c_size_t(ws_bytes),
        _ptr(recv_x, "recv_x", _FP8 if shape.use_fp8 else _BF16, rows * H),
        _scales_ptr(shape, recv_scales, rows), _ptr(recv_src_idx, "recv_src_idx", _I32, rows),
        _ptr(status, "status", _STATUS, 1), _stream(stream, num_tokens_per_expert))
    if rc != EP_OK:
        raise EpError(rc, "ep_layout_dispatch")


def _scales_ptr(shape: ep_shape, recv_scales, rows: int):
    if not shape.use_fp8:
        return None
    types = _STATUS if shape.scale_format == EP_SCALE_UE8M0 else _F32
    return _ptr(recv_scales, "recv_scales", types, rows * scale_row_elems(shape))


def ep_dispatch_expand(shape: ep_shape, x: torch.Tensor, topk_idx: torch.Tensor,
                       expert_slot: torch.Tensor, expert_offset: torch.Tensor,
                       num_tokens_per_expert: torch.Tensor, recv_x: torch.Tensor,
                       recv_scales: Optional[torch.Tensor], recv_src_idx: torch.Tensor,
                       status: Optional[torch.Tensor] = None, stream=None) -> None:
    """Dispatch pack into the expand layout; see ``ep_dispatch_expand`` in include/ep.h."""
    N, H, K, E = shape.num_tokens, shape.hidden, shape.num_topk, shape.num_experts
    T = expand_rows(shape)
    rc = _call("ep_dispatch_expand", 
        ctypes.byref(shape), _ptr(x, "x", _BF16, N * H), _ptr(topk_idx, "topk_idx", _I64, N * K),
        _ptr(expert_slot, "expert_slot", _I32, N * K),
        _ptr(expert_offset, "expert_offset", _I32, E + 1),
        _ptr(num_tokens_per_expert, "num_tokens_per_expert", _I32, E),
        _ptr(recv_x, "recv_x", _FP8 if shape.use_fp8 else _BF16, T * H),
        _scales_ptr(shape, recv_scales, T), _ptr(recv_src_idx, "recv_src_idx", _I32, T),
        _ptr(status, "status", _STATUS, 1), _stream(stream, recv_x))
    if rc != EP_OK:
        raise EpError(rc, "ep_dispatch_expand")


def ep_combine_expand(shape: ep_shape, expert_out: torch.Tensor, topk_idx: torch.Tensor,
                      topk_weights: torch.Tensor, expert_slot: torch.Tensor,
                      expert_offset: torch.Tensor, combined_x: torch.Tensor,
                      status: Optional[torch.Tensor] = None, stream=None,
                      bias: Optional[torch.Tensor] = None) -> None:
    """Combine from the expand layout; see ``ep_combine_expand`` in include/ep.h."""
    N, H, K, E = shape.num_tokens, shape.hidden, shape.num_topk, shape.num_experts
    rc = _call("ep_combine_expand", 
        ctypes.byref(shape), _ptr(expert_out, "expert_out", _BF16, expand_rows(shape) * H),
        _ptr(topk_idx, "topk_idx", _I64, N * K), _ptr(topk_weights, "topk_weights", _F32, N * K),
        _ptr(expert_slot, "expert_slot", _I32, N * K),
        _ptr(expert_offset, "expert_offset", _I32, E + 1), _ptr(bias, "bias", _BF16, N * H),
        _ptr(combined_x, "combined_x", _BF16, N * H), _ptr(status, "status", _STATUS, 1),
        _stream(stream, combined_x))
    if rc != EP_OK:
        raise EpError(rc, "ep_combine_expand")


def ep_dispatch_normal(shape: ep_shape, x: torch.Tensor, topk_idx: torch.Tensor,
                       topk_weights: Optional[torch.Tensor], rank_slot: torch.Tensor,
                       recv_x: torch.Tensor, recv_scales: Optional[torch.Tensor],
                       recv_topk_idx: torch.Tensor, recv_topk_weights: Optional[torch.Tensor],
                       recv_src_idx: torch.Tensor, status: Optional[torch.Tensor] = None,
                       stream=None) -> None:
    """Normal-mode dispatch; see ``ep_dispatch_normal`` in include/ep.h."""
    N, H, K, R = shape.num_tokens, shape.hidden, shape.num_topk, shape.num_ranks
    rows = R * shape.num_max_dispatch_tokens_per_rank
    rc = _call("ep_dispatch_normal", 
        ctypes.byref(shape), _ptr(x, "x", _BF16, N * H), _ptr(topk_idx, "topk_idx", _I64, N * K),
        _ptr(topk_weights, "topk_weights", _F32, N * K), _ptr(rank_slot, "rank_slot", _I32, N * R),
        _ptr(recv_x, "recv_x", _FP8 if shape.use_fp8 else _BF16, rows * H),
        _scales_ptr(shape, recv_scales, rows),
        _ptr(recv_topk_idx, "recv_topk_idx", _I64, rows * K),
        _ptr(recv_topk_weights, "recv_topk_weights", _F32, rows * K),
        _ptr(recv_src_idx, "recv_src_idx", _I32, rows), _ptr(status, "status", _STATUS, 1),
        _stream(stream, recv_x))
    if rc != EP_OK:
        raise EpError(rc, "ep_dispatch_normal")


def ep_combine_normal(shape: ep_shape, x: torch.Tensor, rank_slot: torch.Tensor,
                      recv_topk_weights: Optional[torch.Tensor], combined_x: torch.Tensor,
                      combined_topk_weights: Optional[torch.Tensor] = None,
                      status: Optional[torch.Tensor] = None, stream=None,
                      bias: Optional[torch.Tensor] = None) -> None:
    """Normal-mode combine; see ``ep_combine_normal`` in include/ep.h."""
    N, H, K, R = shape.num_tokens, shape.hidden, shape.num_topk, shape.num_ranks
    rows = R * shape.num_max_dispatch_tokens_per_rank
    rc = _call("ep_combine_normal", 
        ctypes.byref(shape), _ptr(x, "x", _BF16, rows * H), _ptr(rank_slot, "rank_slot", _I32, N * R),
        _ptr(recv_topk_weights, "recv_topk_weights", _F32, rows * K),
        _ptr(bias, "bias", _BF16, N * H), _ptr(combined_x, "combined_x", _BF16, N * H),
        _ptr(combined_topk_weights, "combined_topk_weights", _F32, N * K),
        _ptr(status, "status", _STATUS, 1), _stream(stream, combined_x))
    if rc != EP_OK:
        raise EpError(rc, "ep_combine_normal")


def ep_combine(shape: ep_shape, expert_out: torch.Tensor, topk_idx: torch.Tensor,
               topk_weights: torch.Tensor, expert_slot: torch.Tensor, combined_x: torch.Tensor,
               status: Optional[torch.Tensor] = None, stream=None,
               bias: Optional[torch.Tensor] = None) -> None:
    """Combine; see ``ep_combine`` in include/ep.h."""
    N, H, K, E, S = shape.num_tokens, shape.hidden, shape.num_topk, shape.num_experts, \
        shape.expert_capacity
    rc = _call("ep_combine", 
        ctypes.byref(shape), _ptr(expert_out, "expert_out", _BF16, E * S * H),
        _ptr(topk_idx, "topk_idx", _I64, N * K), _ptr(topk_weights, "topk_weights", _F32, N * K),
        _ptr(expert_slot, "expert_slot", _I32, N * K), _ptr(bias, "bias", _BF16, N * H),
        _ptr(combined_x, "combined_x", _BF16, N * H), _ptr(status, "status", _STATUS, 1),
        _stream(stream, combined_x))
    if rc != EP_OK:
        raise EpError(rc, "ep_combine")


def ep_group_limited_topk(shape: ep_shape, num_groups: int, topk_groups: int, rule: int,
                          scores: torch.Tensor, topk_idx: torch.Tensor,
                          topk_weights: Optional[torch.Tensor] = None, stream=None) -> None:
    """Group-limited top-k gating under ``rule`` (EP_GATE_MAX_SOFTMAX or
    EP_GATE_SUM_SIGMOID); see ``ep_group_limited_topk`` in include/ep.h."""
    N, E, K = shape.num_tokens, shape.num_experts, shape.num_topk
    rc = _call("ep_group_limited_topk", 
        ctypes.byref(shape), ctypes.c_int32(int(num_groups)), ctypes.c_int32(int(topk_groups)),
        ctypes.c_int32(int(rule)), _ptr(scores, "scores", _F32, N * E), _ptr(topk_idx, "topk_idx", _I64, N * K),
        _ptr(topk_weights, "topk_weights", _F32, N * K), _stream(stream, topk_idx))
    if rc != EP_OK:
        raise EpError(rc, "ep_group_limited_topk")


def ep_logfmt_encode(shape: ep_shape, expert_out: torch.Tensor, topk_idx: torch.Tensor,
                     expert_slot: torch.Tensor, codes: torch.Tensor, headers: torch.Tensor,
                     status: Optional[torch.Tensor] = None, stream=None) -> None:
    """LogFMT encoding of the routed expert-output rows; see
    ``ep_logfmt_encode`` in include/ep.h."""
    N, H, K, E, S = (shape.num_tokens, shape.hidden, shape.num_topk, shape.num_experts,
                     shape.expert_capacity)
    rc = _call("ep_logfmt_encode", 
        ctypes.byref(shape), _ptr(expert_out, "expert_out", _BF16, E * S * H),
        _ptr(topk_idx, "topk_idx", _I64, N * K), _ptr(expert_slot, "expert_slot", _I32, N * K),
        _ptr(codes, "codes", (torch.uint8,), E * S * H),
        _ptr(headers, "headers", _F32, E * S * (H // 128) * 2), _ptr(status, "status", _STATUS, 1),
        _stream(stream, codes))
    if rc != EP_OK:
        raise EpError(rc, "ep_logfmt_encode")


def ep_combine_logfmt(shape: ep_shape, codes: torch.Tensor, headers: torch.Tensor,
                      topk_idx: torch.Tensor, topk_weights: torch.Tensor, expert_slot: torch.Tensor,
                      combined_x: torch.Tensor, status: Optional[torch.Tensor] = None, stream=None,
                      bias: Optional[torch.Tensor] = None) -> None:
    """Combine of LogFMT expert outputs; see ``ep_combine_logfmt`` in
    include/ep.h."""
    N, H, K, E, S = (shape.num_tokens, shape.hidden, shape.num_topk, shape.num_experts,
                     shape.expert_capacity)
    rc = _call("ep_combine_logfmt", 
        ctypes.byref(shape), _ptr(codes, "codes", (torch.uint8,), E * S * H),
        _ptr(headers, "headers", _F32, E * S * (H // 128) * 2),
        _ptr(topk_idx, "topk_idx", _I64, N * K), _ptr(topk_weights, "topk_weights", _F32, N * K),
        _ptr(expert_slot, "expert_slot", _I32, N * K), _ptr(bias, "bias", _BF16, N * H),
        _ptr(combined_x, "combined_x", _BF16, N * H), _ptr(status, "status", _STATUS, 1),
        _stream(stream, combined_x))
    if rc != EP_OK:
        raise EpError(rc, "ep_combine_logfmt")


def ep_probe_log2_bf16(bits: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    """The LogFMT encoder's rounded log2 over an array of bf16 patterns; see
    include/ep_probe.h."""
    n = bits.numel()
    rc = _call("ep_probe_log2_bf16", _ptr(bits, "bits", _BF16), _ptr(out, "out", _F32, n),
                                  ctypes.c_int64(n), _stream(stream, bits))
    if rc != EP_OK:
        raise EpError(rc, "ep_probe_log2_bf16")


def ep_probe_e4m3fn(values: torch.Tensor, out_hw: Optional[torch.Tensor],
                    out_sw: Optional[torch.Tensor], stream=None) -> None:
    """The pack's clamp + FP8 conversion over an array; see include/ep_probe.h."""
    n = values.numel()
    rc = _call("ep_probe_e4m3fn", _ptr(values, "values", _F32), _ptr(out_hw, "out_hw", _U8, n),
                               _ptr(out_sw, "out_sw", _U8, n), ctypes.c_int64(n),
                               _stream(stream, values))
    if rc != EP_OK:
        raise EpError(rc, "ep_probe_e4m3fn")


def allocate(shape: ep_shape, device="cuda", parts=("layout", "dispatch", "combine")) -> dict:
    """torch.empty buffers for the outputs of the requested parts of the path
    ("layout", "dispatch", "combine", "expert_out", and for the other receive
    layouts "normal" and "expand"), sized as ep_query_sizes says.  Contents
    are uninitialised except ``status`` (zero)."""
    sz = ep_query_sizes(shape)
    N, H, K, E, R, S = (shape.num_tokens, shape.hidden, shape.num_topk, shape.num_experts,
                        shape.num_ranks, shape.expert_capacity)
    dev = torch.device(device)
    out = {"status": torch.zeros(1, dtype=torch.int32, device=dev)}
    if "layout" in parts:
        out.update({
            "num_tokens_per_rank": torch.empty(R, dtype=torch.int32, device=dev),
            "num_tokens_per_expert": torch.empty(E, dtype=torch.int32, device=dev),
            "is_token_in_rank": torch.empty((N, R), dtype=torch.uint8, device=dev),
            "expert_slot": torch.empty((N, K), dtype=torch.int32, device=dev),
            "rank_slot": torch.empty((N, R), dtype=torch.int32, device=dev),
            "expert_offset": torch.empty(E + 1, dtype=torch.int32, device=dev),
            "workspace": (torch.empty(sz["layout_workspace"], dtype=torch.uint8, device=dev)
                          if sz["layout_workspace"] else None),
        })
    if "dispatch" in parts:
        out.update({
            "recv_x": torch.empty((E, S, H), dtype=torch.uint8 if shape.use_fp8 else torch.int16,
                                  device=dev),
            "recv_scales": (None if not shape.use_fp8 else
                            torch.empty((E, S, (H // 128 + 3) // 4), dtype=torch.int32, device=dev)
                            if shape.scale_format == EP_SCALE_UE8M0 else
                            torch.empty((E, S, H // 128), dtype=torch.float32, device=dev)),
            "recv_src_idx": torch.empty((E, S), dtype=torch.int32, device=dev),
        })
    if "combine" in parts:
        out["combined_x"] = torch.empty((N, H), dtype=torch.int16, device=dev)
    if "logfmt" in parts:
        out.update({
            "logfmt_codes": torch.empty((E, S, H), dtype=torch.uint8, device=dev),
            "logfmt_headers": torch.empty((E, S, H // 128, 2), dtype=torch.float32, device=dev),
        })
    if "expert_out" in parts:
        out["expert_out"] = torch.empty((E, S, H), dtype=torch.int16, device=dev)
    rx_dtype = torch.uint8 if shape.use_fp8 else torch.int16
    sc_dtype = torch.int32 if shape.scale_format == EP_SCALE_UE8M0 else torch.float32
    G = scale_row_elems(shape)
    if "normal" in parts:
        M = shape.num_max_dispatch_tokens_per_rank
        out.update({
            "recv_x_normal": torch.empty((R, M, H), dtype=rx_dtype, device=dev),
            "recv_scales_normal": (torch.empty((R, M, G), dtype=sc_dtype, device=dev)
                                   if shape.use_fp8 else None),
            "recv_topk_idx": torch.empty((R, M, K), dtype=torch.int64, device=dev),
            "recv_topk_weights": torch.empty((R, M, K), dtype=torch.float32, device=dev),
            "recv_src_idx_normal": torch.empty((R, M), dtype=torch.int32, device=dev),
            "combined_topk_weights": torch.empty((N, K), dtype=torch.float32, device=dev),
        })
    if "expand" in parts:
        T = expand_rows(shape)
        out.update({
            "recv_x_expand": torch.empty((T, H), dtype=rx_dtype, device=dev),
            "recv_scales_expand": (torch.empty((T, G), dtype=sc_dtype, device=dev)
                                   if shape.use_fp8 else None),
            "recv_src_idx_expand": torch.empty(T, dtype=torch.int32, device=dev),
        })
    return out


# ---- the path in three calls, allocating with torch --------------------------
def _on_stream(stream):
    """Context in which torch allocates (and fills) on the stream the library
    launches on, so the caching allocator orders every reuse of these blocks
    after the launches that use them: ``stream`` may be None (torch's current
    stream), a torch stream, or a raw hipStream_t handle."""
    if stream is None:
        return contextlib.nullcontext()
    if not isinstance(stream, torch.cuda.Stream):
        stream = torch.cuda.ExternalStream(int(stream))
    return torch.cuda.stream(stream)


@dataclasses.dataclass
class Handle:
    """The layout of one routing, reused by its dispatch and combine (the
    handle the pages' dispatch returns for the combine): the shape without a
    hidden size, the routing itself and every layout output."""
    shape: ep_shape
    topk_idx: torch.Tensor
    num_tokens_per_rank: torch.Tensor
    num_tokens_per_expert: torch.Tensor
    is_token_in_rank: torch.Tensor
    expert_slot: torch.Tensor
    rank_slot: torch.Tensor
    expert_offset: torch.Tensor
    status: torch.Tensor

    def with_hidden(self, hidden: int, use_fp8: bool = False,
                    scale_format: int = EP_SCALE_FP32) -> ep_shape:
        s = self.shape
        return make_shape(s.num_tokens, hidden, s.num_topk, s.num_experts, s.num_ranks,
                          s.num_max_dispatch_tokens_per_rank, s.expert_capacity, use_fp8,
                          scale_format if use_fp8 else EP_SCALE_FP32, s.expert_alignment)


def layout(topk_idx: torch.Tensor, num_experts: int, num_ranks: int,
           num_max_dispatch_tokens_per_rank: Optional[int] = None,
           expert_capacity: Optional[int] = None, expert_alignment: int = 0,
           stream=None) -> Handle:
    """``ep_layout`` on a [N, K] int64 routing (-1 = masked), outputs allocated
    here on ``stream`` (torch's current stream when None).  M defaults to N
    and the expert capacity S to M."""
    N, K = topk_idx.shape
    M = max(N, 1) if num_max_dispatch_tokens_per_rank is None else num_max_dispatch_tokens_per_rank
    S = M if expert_capacity is None else expert_capacity
    # the layout reads no activations: any valid hidden size will do here
    shape = make_shape(N, 8, K, num_experts, num_ranks, M, S, False, EP_SCALE_FP32, expert_alignment)
    with _on_stream(stream):
        b = allocate(shape, topk_idx.device, parts=("layout",))
        ep_layout(shape, topk_idx, b["num_tokens_per_rank"], b["num_tokens_per_expert"],
                  b["is_token_in_rank"], b["expert_slot"], b["rank_slot"], b["expert_offset"],
                  b["workspace"], b["status"], stream=stream)
    return Handle(shape, topk_idx, b["num_tokens_per_rank"], b["num_tokens_per_expert"],
                  b["is_token_in_rank"], b["expert_slot"], b["rank_slot"], b["expert_offset"],
                  b["status"])


def dispatch(x: torch.Tensor, handle: Handle, use_fp8: bool = True,
             scale_format: int = EP_SCALE_FP32, stream=None):
    """``ep_dispatch`` of bf16 ``x`` [N, H] by a layout's handle.  Returns
    (recv_x [E, S, H] as float8_e4m3fn or bfloat16, recv_scales [E, S, H/128]
    fp32 (int32 words for UE8M0) or None, recv_src_idx [E, S]), allocated on
    ``stream``; rows at or past num_tokens_per_expert[e] are unwritten."""
    shape = handle.with_hidden(x.shape[1], use_fp8, scale_format)
    with _on_stream(stream):
        b = allocate(shape, x.device, parts=("dispatch",))
        ep_dispatch(shape, x, handle.topk_idx, handle.expert_slot, b["recv_x"], b["recv_scales"],
                    b["recv_src_idx"], handle.status, stream=stream)
    recv_x = b["recv_x"].view(torch.float8_e4m3fn if use_fp8 else torch.bfloat16)
    return recv_x, b["recv_scales"], b["recv_src_idx"]


def combine(expert_out: torch.Tensor, handle: Handle, topk_weights: torch.Tensor,
            bias: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """``ep_combine`` of bf16 expert outputs [E, S, H] by a layout's handle:
    returns the [N, H] bfloat16 weighted sums in token order (plus ``bias``),
    allocated on ``stream``."""
    s = handle.shape
    if expert_out.dim() != 3 or tuple(expert_out.shape[:2]) != (s.num_experts, s.expert_capacity):
        raise ValueError(f"expert_out has shape {tuple(expert_out.shape)}, expected "
                         f"[{s.num_experts}, {s.expert_capacity}, H]")
    shape = handle.with_hidden(expert_out.shape[-1])
    with _on_stream(stream):
        out = torch.empty((shape.num_tokens, shape.hidden), dtype=torch.bfloat16,
                          device=expert_out.device)
        ep_combine(shape, expert_out, handle.topk_idx, topk_weights, handle.expert_slot, out,
                   handle.status, stream=stream, bias=bias)
    return out
