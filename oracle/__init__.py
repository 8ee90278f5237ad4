"""CPU oracle for the MoE expert-parallel dispatch layout, dispatch pack and combine.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU library
(``combine_ep_layout_02_amd``) never imports it and shares no code with it.

The arithmetic lives in ``ep_oracle.c`` (plain single-threaded C, gcc -O2, no
fast-math, no FP contraction).  This module only marshals numpy arrays into
that library through ctypes.  Each function's docstring names the passage of
the DeepEP pages it follows; the C source restates the definition.

Pins (what ties the oracle to something other than itself) are in
``tests/pins.py``; every function here is pinned, none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "ep_oracle.c")
LIBRARY = os.path.join(_HERE, "libep_oracle.so")

# gcc flags: IEEE binary32 arithmetic in source order, no fused contraction.
CFLAGS = ["-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]

STATUS_OK = 0
STATUS_BAD_EXPERT_ID = 1
STATUS_BAD_SLOT = 2
STATUS_BAD_ARGS = 4

GATE_MAX_SOFTMAX = 0
GATE_SUM_SIGMOID = 1


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle with gcc into a shared library and return its path."""
    subprocess.check_call(["gcc", *CFLAGS, "-o", output, source, "-lm"])
    return output


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """ctypes handle on one build of ``ep_oracle.c`` (the default build, or a
    planted-mistake variant built by the mutation tests)."""

    def __init__(self, path: str = LIBRARY):
        self.path = path
        lib = ctypes.CDLL(path)
        i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        lib.oracle_layout.argtypes = [i32, i32, i32, i32] + [vp] * 7
        lib.oracle_layout.restype = ctypes.c_int
        lib.oracle_pack.argtypes = [i32] * 6 + [vp] * 6
        lib.oracle_pack.restype = ctypes.c_int
        lib.oracle_combine.argtypes = [i32] * 5 + [vp] * 6
        lib.oracle_combine.restype = ctypes.c_int
        lib.oracle_e4m3fn_encode_array.argtypes = [i64, vp, vp]
        lib.oracle_e4m3fn_decode_array.argtypes = [i64, vp, vp]
        lib.oracle_bf16_rne_array.argtypes = [i64, vp, vp]
        lib.oracle_quantize_rows.argtypes = [i32, i32, vp, vp, vp]
        lib.oracle_dequant_rows.argtypes = [i32, i32, vp, vp, vp]
        lib.oracle_pack_fmt.argtypes = [i32] * 7 + [vp] * 6
        lib.oracle_pack_fmt.restype = ctypes.c_int
        lib.oracle_quantize_rows_pow2.argtypes = [i32, i32, vp, vp, vp]
        lib.oracle_pow2_scale_exponent.argtypes = [ctypes.c_float]
        lib.oracle_pow2_scale_exponent.restype = ctypes.c_int
        lib.oracle_aligned_offsets.argtypes = [i32, vp, i32, vp]
        lib.oracle_pack_expand.argtypes = [i32] * 7 + [vp] * 8
        lib.oracle_pack_expand.restype = ctypes.c_int
        lib.oracle_combine_expand.argtypes = [i32] * 5 + [vp] * 7
        lib.oracle_combine_expand.restype = ctypes.c_int
        lib.oracle_dispatch_normal.argtypes = [i32] * 8 + [vp] * 9
        lib.oracle_dispatch_normal.restype = ctypes.c_int
        lib.oracle_combine_normal.argtypes = [i32] * 5 + [vp] * 6
        lib.oracle_combine_normal.restype = ctypes.c_int
        lib.oracle_group_limited_topk.argtypes = [i32] * 6 + [vp] * 3
        lib.oracle_timed_path.argtypes = [i32] * 7 + [vp] * 15
        lib.oracle_log2_rn_array.argtypes = [i64, vp, vp]
        lib.oracle_logfmt_encode_rows.argtypes = [i64, i32, vp, vp, vp]
        lib.oracle_logfmt_decode_rows.argtypes = [i64, i32, vp, vp, vp]
        lib.oracle_combine_logfmt.argtypes = [i32] * 5 + [vp] * 7
        lib.oracle_combine_logfmt.restype = ctypes.c_int
        lib.oracle_timed_path.restype = ctypes.c_int
        lib.oracle_group_limited_topk.restype = ctypes.c_int
        self.lib = lib

    # ------------------------------------------------------------- layout
    def layout(self, topk_idx: np.ndarray, num_experts: int, num_ranks: int,
               alignment: int = 1) -> dict:
        """Dispatch layout (DeepEP V1 Legacy guide §5.2(1); Ascend deep dive,
        "Dispatch's Three Phases", phase 2).  ``topk_idx`` int64 [N, K] with -1
        for masked entries.  Returns counts, mask, slots, offsets, status;
        with ``alignment`` A > 1 the offsets are those of the expand layout
        (each queue rounded up to a multiple of A; phase 1)."""
        idx = np.ascontiguousarray(topk_idx, dtype=np.int64)
        n, k = idx.shape
        e, r = int(num_experts), int(num_ranks)
        out = {
            "num_tokens_per_rank": np.empty(r, np.int32),
            "num_tokens_per_expert": np.empty(e, np.int32),
            "is_token_in_rank": np.empty((n, r), np.uint8),
            "expert_slot": np.empty((n, k), np.int32),
            "rank_slot": np.empty((n, r), np.int32),
            "expert_offset": np.empty(e + 1, np.int32),
        }
        st = self.lib.oracle_layout(
            n, k, e, r, _ptr(idx), _ptr(out["num_tokens_per_rank"]),
            _ptr(out["num_tokens_per_expert"]), _ptr(out["is_token_in_rank"]),
            _ptr(out["expert_slot"]), _ptr(out["rank_slot"]), _ptr(out["expert_offset"]))
        out["status"] = int(st)
        if alignment > 1:
            out["expert_offset"] = self.aligned_offsets(out["num_tokens_per_expert"], alignment)
        return out

    def aligned_offsets(self, counts: np.ndarray, alignment: int) -> np.ndarray:
        """Expand-layout queue starts (Ascend deep dive, "Dispatch's Three
        Phases", phase 1: queues padded to a multiple of the alignment)."""
        c = np.ascontiguousarray(counts, dtype=np.int32)
        out = np.empty(c.size + 1, np.int32)
        self.lib.oracle_aligned_offsets(c.size, _ptr(c), int(alignment), _ptr(out))
        return out

    # --------------------------------------------------------------- pack
    def pack(self, x_bits: np.ndarray, topk_idx: np.ndarray, expert_slot: np.ndarray,
             num_experts: int, capacity: int, use_fp8: bool, fill: int = 0, scale_format: int = 0):
        """Dispatch pack (Lesson 14 §3 receive shape; DeepEP V1 Legacy guide
        §5.2(6) and §6.3 FP8 with one scale per 128 channels; §6.3
        round_scale / use_ue8m0 for scale_format 1 / 2).  ``x_bits`` is the
        bf16 bit pattern, uint16 [N, H].  Returns (recv_x, recv_scales,
        recv_src_idx, status) with recv_x uint8 [E, S, H] (FP8) or uint16
        [E, S, H] (BF16); recv_scales float32 [E, S, H/128] (formats 0, 1) or
        uint32 [E, S, ceil(H/512)] (format 2, four UE8M0 bytes per word);
        rows never written keep ``fill``."""
        x = np.ascontiguousarray(x_bits, dtype=np.uint16)
        idx = np.ascontiguousarray(topk_idx, dtype=np.int64)
        slot = np.ascontiguousarray(expert_slot, dtype=np.int32)
        n, h = x.shape
        k = idx.shape[1]
        e, s = int(num_experts), int(capacity)
        g = h // 128
        if use_fp8:
            recv_x = np.full((e, s, h), fill & 0xFF, np.uint8)
            if scale_format == 2:
                recv_scales = np.full((e, s, (g + 3) // 4), 0xDEADBEEF, np.uint32)
            else:
                recv_scales = np.full((e, s, g), np.nan, np.float32)
        else:
            recv_x = np.full((e, s, h), fill & 0xFFFF, np.uint16)
            recv_scales = None
        recv_src = np.full((e, s), -2, np.int32)
        st = self.lib.oracle_pack_fmt(n, h, k, e, s, int(bool(use_fp8)), int(scale_format),
                                      _ptr(x), _ptr(idx), _ptr(slot), _ptr(recv_x),
                                      _ptr(recv_scales), _ptr(recv_src))
        return recv_x, recv_scales, recv_src, int(st)

    @staticmethod
    def _recv_buffers(rows: int, h: int, use_fp8: bool, scale_format: int, fill: int):
        g = h // 128
        if use_fp8:
            recv_x = np.full((rows, h), fill & 0xFF, np.uint8)
            if scale_format == 2:
                recv_scales = np.full((rows, (g + 3) // 4), 0xDEADBEEF, np.uint32)
            else:
                recv_scales = np.full((rows, g), np.nan, np.float32)
        else:
            recv_x = np.full((rows, h), fill & 0xFFFF, np.uint16)
            recv_scales = None
        return recv_x, recv_scales

    def pack_expand(self, x_bits: np.ndarray, topk_idx: np.ndarray, expert_slot: np.ndarray,
                    expert_offset: np.ndarray, counts: np.ndarray, rows: int, use_fp8: bool,
                    fill: int = 0, scale_format: int = 0):
        """Dispatch pack into the expand layout (Ascend deep dive, "Dispatch's
        Three Phases", phase 1).  One buffer of ``rows`` rows; returns
        (recv_x [rows, H], recv_scales, recv_src_idx [rows], status); rows at
        or past expert_offset[E] keep ``fill`` (-2 for the source index)."""
        x = np.ascontiguousarray(x_bits, dtype=np.uint16)
        idx = np.ascontiguousarray(topk_idx, dtype=np.int64)
        slot = np.ascontiguousarray(expert_slot, dtype=np.int32)
        off = np.ascontiguousarray(expert_offset, dtype=np.int32)
        cnt = np.ascontiguousarray(counts, dtype=np.int32)
        n, h = x.shape
        k = idx.shape[1]
        e = cnt.size
        recv_x, recv_scales = self._recv_buffers(rows, h, use_fp8, scale_format, fill)
        recv_src = np.full(rows, -2, np.int32)
        st = self.lib.oracle_pack_expand(n, h, k, e, int(rows), int(bool(use_fp8)),
                                         int(scale_format), _ptr(x), _ptr(idx), _ptr(slot),
                                         _ptr(off), _ptr(cnt), _ptr(recv_x), _ptr(recv_scales),
                                         _ptr(recv_src))
        return recv_x, recv_scales, recv_src, int(st)

    def combine_expand(self, y_bits: np.ndarray, topk_idx: np.ndarray, topk_weights: np.ndarray,
                       expert_slot: np.ndarray, expert_offset: np.ndarray,
                       bias: np.ndarray | None = None):
        """Combine from expert outputs in the expand layout, y_bits [rows, H]."""
        y = np.ascontiguousarray(y_bits, dtype=np.uint16)
        idx = np.ascontiguousarray(topk_idx, dtype=np.int64)
        w = np.ascontiguousarray(topk_weights, dtype=np.float32)
        slot = np.ascontiguousarray(expert_slot, dtype=np.int32)
        off = np.ascontiguousarray(expert_offset, dtype=np.int32)
        n, k = idx.shape
        rows, h = y.shape
        out = np.empty((n, h), np.uint16)
        b = self._bias(bias, n, h)
        st = self.lib.oracle_combine_expand(n, h, k, off.size - 1, rows, _ptr(y), _ptr(idx),
                                            _ptr(w), _ptr(slot), _ptr(off), _ptr(b), _ptr(out))
        return out, int(st)

    def dispatch_normal(self, x_bits: np.ndarray, topk_idx: np.ndarray,
                        topk_weights: np.ndarray | None, rank_slot: np.ndarray, num_experts: int,
                        num_ranks: int, rows_per_rank: int, use_fp8: bool, fill: int = 0,
                        scale_format: int = 0):
        """Normal-mode dispatch (DeepEP V1 Legacy guide §5.1): one row per
        (token, rank) in rank-major buffers [R, M, ...].  Returns a dict with
        recv_x, recv_scales, recv_topk_idx [R, M, K], recv_topk_weights
        [R, M, K] (None without weights), recv_src_idx [R, M] and status;
        unwritten rows keep ``fill`` (-2 / -7 / NaN for the metadata)."""
        x = np.ascontiguousarray(x_bits, dtype=np.uint16)
        idx = np.ascontiguousarray(topk_idx, dtype=np.int64)
        rs = np.ascontiguousarray(rank_slot, dtype=np.int32)
        n, h = x.shape
        k = idx.shape[1]
        r, m = int(num_ranks), int(rows_per_rank)
        recv_x, recv_scales = self._recv_buffers(r * m, h, use_fp8, scale_format, fill)
        out = {
            "recv_x": recv_x.reshape(r, m, h),
            "recv_scales": None if recv_scales is None else recv_scales.reshape(r, m, -1),
            "recv_topk_idx": np.full((r, m, k), -7, np.int64),
            "recv_topk_weights": None,
            "recv_src_idx": np.full((r, m), -2, np.int32),
        }
        w = None
        if topk_weights is not None:
            w = np.ascontiguousarray(topk_weights, dtype=np.float32)
            out["recv_topk_weights"] = np.full((r, m, k), np.nan, np.float32)
        st = self.lib.oracle_dispatch_normal(
            n, h, k, int(num_experts), r, m, int(bool(use_fp8)), int(scale_format), _ptr(x),
            _ptr(idx), _ptr(w), _ptr(rs), _ptr(recv_x), _ptr(recv_scales),
            _ptr(out["recv_topk_idx"]), _ptr(out["recv_topk_weights"]), _ptr(out["recv_src_idx"]))
        out["status"] = int(st)
        return out

    def combine_normal(self, y_bits: np.ndarray, rank_slot: np.ndarray,
                       recv_topk_weights: np.ndarray | None = None,
                       bias: np.ndarray | None = None):
        """Normal-mode combine (DeepEP V1 Legacy guide §5.1): y_bits [R, M, H]
        one row per received token; returns (combined bf16 bits [N, H],
        combined topk weights [N, K] or None, status)."""
        y = np.ascontiguousarray(y_bits, dtype=np.uint16)
        rs = np.ascontiguousarray(rank_slot, dtype=np.int32)
        r, m, h = y.shape
        n = rs.shape[0]
        out = np.empty((n, h), np.uint16)
        rw, cw, k = None, None, 1
        if recv_topk_weights is not None:
            rw = np.ascontiguousarray(recv_topk_weights, dtype=np.float32)
            k = rw.shape[-1]
            cw = np.empty((n, k), np.float32)
        b = self._bias(bias, n, h)
        st = self.lib.oracle_combine_normal(n, h, k, r, m, _ptr(y), _ptr(rs), _ptr(rw), _ptr(b),
                                            _ptr(out), _ptr(cw))
        return out, cw, int(st)

    def group_limited_topk(self, scores: np.ndarray, num_groups: int, topk_groups: int,
                           num_topk: int, rule: int = 0):
        """Group-limited top-k gating (DeepEP V1 Legacy guide §1 and §2.1;
        Lesson 14 §3 Q3 and exercise).  ``scores`` float32 [N, E]; ``rule``
        GATE_MAX_SOFTMAX (group score = best expert, softmax weights) or
        GATE_SUM_SIGMOID (group score = ordered binary32 sum, normalised
        sigmoid weights).  Returns (topk_idx int64 [N, K], topk_weights
        float32 [N, K], status)."""
        sc = np.ascontiguousarray(scores, dtype=np.float32)
        n, e = sc.shape
        k = int(num_topk)
        idx = np.empty((n, k), np.int64)
        w = np.empty((n, k), np.float32)
        st = self.lib.oracle_group_limited_topk(n, e, int(num_groups), int(topk_groups), k,
                                                int(rule), _ptr(sc), _ptr(idx), _ptr(w))
        return idx, w, int(st)

    def quantize_rows_pow2(self, x_bits: np.ndarray):
        """Power-of-two-scale FP8 payload of each row: (q uint8 [N, H],
        exponents int32 [N, H/128]); the scale of a block is 2^exponent."""
        x = np.ascontiguousarray(x_bits, dtype=np.uint16)
        n, h = x.shape
        q = np.empty((n, h), np.uint8)
        ex = np.empty((n, h // 128), np.int32)
        self.lib.oracle_quantize_rows_pow2(n, h, _ptr(x), _ptr(q), _ptr(ex))
        return q, ex

    def pow2_scale_exponent(self, amax_floored: float) -> int:
        return int(self.lib.oracle_pow2_scale_exponent(ctypes.c_float(amax_floored)))

    # ------------------------------------------------------------ combine
    @staticmethod
    def _bias(bias, n, h):
        if bias is None:
            return None
        b = np.ascontiguousarray(bias, dtype=np.uint16)
        assert b.shape == (n, h), "bias must be [N, H] bf16 bits"
        return b

    def combine(self, y_bits: np.ndarray, topk_idx: np.ndarray, topk_weights: np.ndarray,
                expert_slot: np.ndarray, num_experts: int, capacity: int,
                bias: np.ndarray | None = None):
        """Combine (Ascend deep dive, "Two Transfers" and "Combine: More
        Output, Same Cost"; Lesson 14 exercise; DeepEP V1 Legacy guide
        §5.2(6)).  ``y_bits`` uint16 [E, S, H] bf16 expert outputs; ``bias``
        optional [N, H] bf16 bits (the shared expert's output, added in the
        epilogue).  Returns (combined bf16 bits uint16 [N, H], status)."""
        y = np.ascontiguousarray(y_bits, dtype=np.uint16)
        idx = np.ascontiguousarray(topk_idx, dtype=np.int64)
        w = np.ascontiguousarray(topk_weights, dtype=np.float32)
        slot = np.ascontiguousarray(expert_slot, dtype=np.int32)
        n, k = idx.shape
        h = y.shape[-1]
        out = np.empty((n, h), np.uint16)
        b = self._bias(bias, n, h)
        st = self.lib.oracle_combine(n, h, k, int(num_experts), int(capacity), _ptr(y),
                                     _ptr(idx), _ptr(w), _ptr(slot), _ptr(b), _ptr(out))
        return out, int(st)

    def timed_path(self, x_bits: np.ndarray, topk_idx: np.ndarray, topk_weights: np.ndarray,
                   expert_out: np.ndarray, num_experts: int, num_ranks: int, capacity: int,
                   use_fp8: bool):
        """The path (layout, pack with fp32 scales, combine of ``expert_out``
        [E, S, H] bf16 bits) on output buffers allocated here, beforehand;
        each phase timed inside the C library.  Returns ((layout_s, pack_s,
        combine_s), status)."""
        x = np.ascontiguousarray(x_bits, dtype=np.uint16)
        idx = np.ascontiguousarray(topk_idx, dtype=np.int64)
        w = np.ascontiguousarray(topk_weights, dtype=np.float32)
        y = np.ascontiguousarray(expert_out, dtype=np.uint16)
        n, h = x.shape
        k = idx.shape[1]
        e, r, s = int(num_experts), int(num_ranks), int(capacity)
        lay = [np.empty(r, np.int32), np.empty(e, np.int32), np.empty((n, r), np.uint8),
               np.empty((n, k), np.int32), np.empty((n, r), np.int32), np.empty(e + 1, np.int32)]
        recv_x = np.empty((e, s, h), np.uint8 if use_fp8 else np.uint16)
        recv_scales = np.empty((e, s, h // 128), np.float32) if use_fp8 else None
        recv_src = np.empty((e, s), np.int32)
        out = np.empty((n, h), np.uint16)
        secs = np.zeros(3, np.float64)
        st = self.lib.oracle_timed_path(n, h, k, e, r, s, int(bool(use_fp8)), _ptr(x), _ptr(idx),
                                        _ptr(w), _ptr(y), *[_ptr(a) for a in lay], _ptr(recv_x),
                                        _ptr(recv_scales), _ptr(recv_src), _ptr(out), _ptr(secs))
        return tuple(float(v) for v in secs), int(st)

    # ------------------------------------------------------------ LogFMT
    def log2_rn(self, a: np.ndarray) -> np.ndarray:
        """log2 of positive floats, rounded to the nearest binary32."""
        v = np.ascontiguousarray(a, dtype=np.float32).ravel()
        out = np.empty_like(v)
        self.lib.oracle_log2_rn_array(v.size, _ptr(v), _ptr(out))
        return out.reshape(np.shape(a))

    def logfmt_encode(self, rows_bits: np.ndarray):
        """LogFMT of bf16 rows uint16 [R, H] (H % 128 == 0; DeepEP V1 Legacy
        guide §6.2: a min/max header per 128 channels, then the data; §7.1
        LogFMT combine): (codes uint8 [R, H], headers float32 [R, H/128, 2]
        holding (lo, hi) per block)."""
        x = np.ascontiguousarray(rows_bits, dtype=np.uint16)
        r, h = x.shape
        codes = np.empty((r, h), np.uint8)
        headers = np.empty((r, h // 128, 2), np.float32)
        self.lib.oracle_logfmt_encode_rows(r, h, _ptr(x), _ptr(codes), _ptr(headers))
        return codes, headers

    def logfmt_decode(self, codes: np.ndarray, headers: np.ndarray) -> np.ndarray:
        """Decoded float32 values [R, H] of LogFMT codes and headers."""
        c = np.ascontiguousarray(codes, dtype=np.uint8)
        hd = np.ascontiguousarray(headers, dtype=np.float32)
        r, h = c.shape
        out = np.empty((r, h), np.float32)
        self.lib.oracle_logfmt_decode_rows(r, h, _ptr(c), _ptr(hd), _ptr(out))
        return out

    def combine_logfmt(self, codes: np.ndarray, headers: np.ndarray, topk_idx: np.ndarray,
                       topk_weights: np.ndarray, expert_slot: np.ndarray, num_experts: int,
                       capacity: int, bias: np.ndarray | None = None):
        """Combine of expert outputs carried as LogFMT: ``codes`` uint8
        [E, S, H], ``headers`` float32 [E, S, H/128, 2].  Returns (combined
        bf16 bits uint16 [N, H], status)."""
        c = np.ascontiguousarray(codes, dtype=np.uint8)
        hd = np.ascontiguousarray(headers, dtype=np.float32)
        idx = np.ascontiguousarray(topk_idx, dtype=np.int64)
        w = np.ascontiguousarray(topk_weights, dtype=np.float32)
        slot = np.ascontiguousarray(expert_slot, dtype=np.int32)
        n, k = idx.shape
        h = c.shape[-1]
        out = np.empty((n, h), np.uint16)
        b = self._bias(bias, n, h)
        st = self.lib.oracle_combine_logfmt(n, h, k, int(num_experts), int(capacity), _ptr(c),
                                            _ptr(hd), _ptr(idx), _ptr(w), _ptr(slot), _ptr(b),
                                            _ptr(out))
        return out, int(st)

    # ------------------------------------------------------------ formats
    def e4m3fn_encode(self, v: np.ndarray) -> np.ndarray:
        a = np.ascontiguousarray(v, dtype=np.float32).ravel()
        out = np.empty(a.size, np.uint8)
        self.lib.oracle_e4m3fn_encode_array(a.size, _ptr(a), _ptr(out))
        return out.reshape(np.shape(v))

    def e4m3fn_decode(self, c: np.ndarray) -> np.ndarray:
        a = np.ascontiguousarray(c, dtype=np.uint8).ravel()
        out = np.empty(a.size, np.float64)
        self.lib.oracle_e4m3fn_decode_array(a.size, _ptr(a), _ptr(out))
        return out.reshape(np.shape(c))

    def bf16_rne(self, v: np.ndarray) -> np.ndarray:
        a = np.ascontiguousarray(v, dtype=np.float32).ravel()
        out = np.empty(a.size, np.uint16)
        self.lib.oracle_bf16_rne_array(a.size, _ptr(a), _ptr(out))
        return out.reshape(np.shape(v))

    def quantize_rows(self, x_bits: np.ndarray):
        """FP8 payload of each row: (q uint8 [N, H], scales float32 [N, H/128])."""
        x = np.ascontiguousarray(x_bits, dtype=np.uint16)
        n, h = x.shape
        q = np.empty((n, h), np.uint8)
        sc = np.empty((n, h // 128), np.float32)
        self.lib.oracle_quantize_rows(n, h, _ptr(x), _ptr(q), _ptr(sc))
        return q, sc

    def dequant_rows(self, q: np.ndarray, scales: np.ndarray) -> np.ndarray:
        """Identity-expert output of FP8 rows: bf16 bits uint16 [N, H]."""
        qq = np.ascontiguousarray(q, dtype=np.uint8)
        sc = np.ascontiguousarray(scales, dtype=np.float32)
        n, h = qq.shape
        y = np.empty((n, h), np.uint16)
        self.lib.oracle_dequant_rows(n, h, _ptr(qq), _ptr(sc), _ptr(y))
        return y


_DEFAULT: Oracle | None = None


def get() -> Oracle:
    """The oracle built from ``ep_oracle.c`` (built with gcc on first use if
    no library is present)."""
    global _DEFAULT
    if _DEFAULT is None:
        if not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
            build()
        _DEFAULT = Oracle(LIBRARY)
    return _DEFAULT
