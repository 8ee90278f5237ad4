"""Plumbing for the GPU tests: move seeded inputs to the device, call the
library through the binding (and so through the C ABI) on poisoned output
buffers, and bring results back as numpy arrays.  No method arithmetic here."""
from __future__ import annotations

import numpy as np
import torch

from combine_ep_layout_02_amd import ep

POISON_I32 = 0x7B7B7B7B
POISON_U8 = 0xEE
POISON_X8 = 0xA5
POISON_X16 = np.int16(np.uint16(0xA5A5).view(np.int16))
POISON_SRC = -2
POISON_SCALE_BITS = 0x7FC0DEAD  # a NaN pattern, set through an int32 view


def say(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    a = t.cpu().numpy()
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    return a


def status_bits(status: torch.Tensor) -> int:
    return int(status.item()) & 0xFFFFFFFF


class LayoutRun:
    """One ep_layout call on poisoned outputs; device tensors kept for reuse."""

    def __init__(self, shape: ep.ep_shape, topk_idx: np.ndarray, stream=None):
        N, K, E, R = shape.num_tokens, shape.num_topk, shape.num_experts, shape.num_ranks
        full = lambda n, v, dt: torch.full((n,), v, dtype=dt, device="cuda")
        self.shape = shape
        self.topk_idx = dev(np.asarray(topk_idx, dtype=np.int64).reshape(N, K))
        self.num_tokens_per_rank = full(R, POISON_I32, torch.int32)
        self.num_tokens_per_expert = full(E, POISON_I32, torch.int32)
        self.is_token_in_rank = full(N * R, POISON_U8, torch.uint8).view(N, R)
        self.expert_slot = full(N * K, POISON_I32, torch.int32).view(N, K)
        self.rank_slot = full(N * R, POISON_I32, torch.int32).view(N, R)
        self.expert_offset = full(E + 1, POISON_I32, torch.int32)
        need = ep.ep_query_sizes(shape)["layout_workspace"]
        self.workspace = full(-(-need // 4), POISON_I32, torch.int32) if need else None
        self.status = torch.zeros(1, dtype=torch.int32, device="cuda")
        ep.ep_layout(shape, self.topk_idx, self.num_tokens_per_rank, self.num_tokens_per_expert,
                     self.is_token_in_rank, self.expert_slot, self.rank_slot, self.expert_offset,
                     self.workspace, self.status, stream=stream)

    def numpy(self) -> dict:
        torch.cuda.synchronize()
        return {
            "num_tokens_per_rank": host(self.num_tokens_per_rank),
            "num_tokens_per_expert": host(self.num_tokens_per_expert),
            "is_token_in_rank": host(self.is_token_in_rank),
            "expert_slot": host(self.expert_slot),
            "rank_slot": host(self.rank_slot),
            "expert_offset": host(self.expert_offset),
            "status": status_bits(self.status),
        }


class DispatchRun:
    """One ep_dispatch call into poisoned receive buffers [E, S, H]."""

    def __init__(self, shape: ep.ep_shape, x_bits: np.ndarray, topk_idx_dev: torch.Tensor,
                 expert_slot_dev: torch.Tensor, x_dev: torch.Tensor | None = None, stream=None):
        E, S, H = shape.num_experts, shape.expert_capacity, shape.hidden
        self.shape = shape
        self.x = dev(x_bits) if x_dev is None else x_dev
        if shape.use_fp8:
            self.recv_x = torch.full((E, S, H), POISON_X8, dtype=torch.uint8, device="cuda")
            if shape.scale_format == ep.EP_SCALE_UE8M0:  # four exponent bytes per word
                self.recv_scales = torch.full((E, S, (H // 128 + 3) // 4), POISON_SCALE_BITS,
                                              dtype=torch.int32, device="cuda")
            else:
                self.recv_scales = torch.full((E, S, H // 128), POISON_SCALE_BITS,
                                              dtype=torch.int32, device="cuda").view(torch.float32)
        else:
            self.recv_x = torch.full((E, S, H), int(POISON_X16), dtype=torch.int16, device="cuda")
            self.recv_scales = None
        self.recv_src_idx = torch.full((E, S), POISON_SRC, dtype=torch.int32, device="cuda")
        self.status = torch.zeros(1, dtype=torch.int32, device="cuda")
        ep.ep_dispatch(shape, self.x, topk_idx_dev, expert_slot_dev, self.recv_x, self.recv_scales,
                       self.recv_src_idx, self.status, stream=stream)


def written_rows(counts: np.ndarray, S: int) -> np.ndarray:
    """Flat row numbers e * S + j for j < min(counts[e], S), in expert order
    (an expert's entries past the capacity S are never written)."""
    return np.concatenate([e * S + np.arange(min(int(c), S), dtype=np.int64)
                           for e, c in enumerate(counts)] + [np.zeros(0, np.int64)])


def gather_rows(t: torch.Tensor, rows: np.ndarray) -> np.ndarray:
    """Rows ``rows`` of a [E, S, ...] device tensor as a host array [P, ...]."""
    nrows = t.shape[0] * t.shape[1]
    if rows.size:
        assert rows.min() >= 0 and rows.max() < nrows, "row index outside the buffer"
    flat = t.reshape(nrows, *t.shape[2:])
    idx = torch.from_numpy(rows).cuda()
    return host(flat.index_select(0, idx))


def unwritten_rows_intact(t: torch.Tensor, counts: np.ndarray, poison: int) -> bool:
    """Every row at or beyond counts[e] of expert e of the integer tensor
    ``t`` [E, S, ...] still holds ``poison``."""
    S = t.shape[1]
    for e, c in enumerate(counts):
        c = int(c)
        if c < S and bool((t[e, c:] != poison).any()):
            return False
    return True


def place_expert_rows(rows_bits: np.ndarray, topk_idx: np.ndarray, expert_slot: np.ndarray,
                      E: int, S: int, H: int) -> torch.Tensor:
    """A [E, S, H] bf16-bits device tensor (poisoned) holding one row per
    valid (t, k) entry, in (t, k) order, at (expert, slot); entries whose slot
    is at or past the capacity S are dropped, as the kernels skip them."""
    y = torch.full((E * S, H), int(POISON_X16), dtype=torch.int16, device="cuda")
    flat_idx = topk_idx.reshape(-1)
    flat_slot = expert_slot.reshape(-1)
    valid = flat_idx >= 0
    keep = flat_slot[valid] < S  # entries past the capacity have no row
    where = flat_idx[valid][keep].astype(np.int64) * S + flat_slot[valid][keep].astype(np.int64)
    if where.size:
        assert where.min() >= 0 and where.max() < E * S, "row index outside the buffer"
        y.index_copy_(0, torch.from_numpy(where).cuda(), dev(rows_bits[keep]))
    return y.view(E, S, H)


def run_combine(shape: ep.ep_shape, y_dev: torch.Tensor, topk_idx_dev: torch.Tensor,
                weights: np.ndarray, expert_slot_dev: torch.Tensor, stream=None,
                bias: np.ndarray | None = None):
    N, H = shape.num_tokens, shape.hidden
    w = dev(np.asarray(weights, dtype=np.float32))
    out = torch.full((N, H), int(POISON_X16), dtype=torch.int16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    b = None if bias is None else dev(bias)
    ep.ep_combine(shape, y_dev, topk_idx_dev, w, expert_slot_dev, out, status, stream=stream,
                  bias=b)
    torch.cuda.synchronize()
    return host(out), status_bits(status)
