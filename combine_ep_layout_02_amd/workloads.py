"""Seeded synthetic inputs for the dispatch layout / pack / combine path.

This module draws inputs only: token activations, top-k routings, router
weights, masks and expert-output rows.  It holds none of the method's
arithmetic (no slot assignment, no quantisation, no reduction), so the GPU
library and the CPU oracle can both be fed from it without sharing code.

The five workloads take the shapes of the DeepEP pages' own benchmarks:

* ``tiny``     64 x 256, 16 experts over 4 ranks, top-2, BF16 (a small case);
* ``decode``   128 x 7168, 256 experts over 8 ranks, top-8, FP8, receive
  buffer [32, 8 * 128, 7168] per rank (DeepEP V1 Legacy guide §2.2, the
  low-latency benchmark; Lesson 14 §3 receive shape);
* ``prefill``  4096 x 7168, 256 experts in 8 groups over 8 ranks, top-4
  groups then top-8 experts, FP8 (DeepEP V1 Legacy guide §2.1, the normal-
  kernel benchmark);
* ``large``    16384 x 7168, 256 experts over 8 ranks, top-6, BF16 (Ascend
  deep dive, "Benchmark Numbers and Caveats" test environment; "Two
  Transfers" gives 1.4 GB per pass for this size);
* ``skewed``   4096 x 4096, 64 experts over 64 ranks, top-6 drawn from a
  Zipf(1.2) popularity, 10 % of entries masked with -1, FP8.

Generator rules (one ``numpy.random.default_rng(1000 + id)`` stream per
workload, drawn in this order: x, routing, weight logits, mask, expert rows):

* x ~ N(0, 1) float32, rounded to bf16 by torch's CPU cast;
* uniform routing: K distinct experts per token, the first K of a random
  permutation (argsort of uniform keys);
* group-limited routing: scores s ~ N(0, 1) [N, E]; group g holds experts
  [g E/G, (g+1) E/G); a group's score is the binary32 sum of its experts'
  scores in ascending expert index from +0; the
  top-4 groups are kept, then the top-K experts by s among them (stable
  order, lowest index first on ties); weights = sigmoid(s_sel) normalised to
  sum 1;
* Zipf routing: popularity p_e proportional to (e+1)^-1.2, K distinct experts
  per token by Gumbel-top-K on log p (equivalent to sequential draws without
  replacement);
* weights (uniform and Zipf routing): softmax over K of N(0, 1) logits;
* mask: exactly floor(fraction * N * K) entries set to -1, chosen by a seeded
  permutation of the flattened entries;
* expert rows: N(0, 1) bf16, one row per valid (t, k) entry in (t, k) order.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    num_tokens: int                       # N
    hidden: int                           # H
    num_topk: int                         # K
    num_experts: int                      # E
    num_ranks: int                        # R (logical EP ranks)
    num_max_dispatch_tokens_per_rank: int  # M
    expert_capacity: int                  # S, rows per expert receive buffer
    use_fp8: bool
    routing: str                          # "uniform" | "group_limited" | "zipf"
    mask_fraction: float = 0.0
    num_groups: int = 0
    topk_groups: int = 0
    zipf_s: float = 0.0

    @property
    def local_experts(self) -> int:
        return self.num_experts // self.num_ranks

    def scaled(self, num_tokens: int, hidden: Optional[int] = None) -> "Workload":
        """The same recipe at another token count (and optionally another
        hidden size).  M becomes max(N, 1) and S keeps its ratio to M."""
        m = max(int(num_tokens), 1)
        s = m * (self.expert_capacity // self.num_max_dispatch_tokens_per_rank)
        return dataclasses.replace(self, num_tokens=int(num_tokens), hidden=hidden or self.hidden,
                                   num_max_dispatch_tokens_per_rank=m, expert_capacity=s)


WORKLOADS = {
    1: Workload(1, "tiny_64x256", 64, 256, 2, 16, 4, 64, 64, False, "uniform"),
    2: Workload(2, "decode_128x7168", 128, 7168, 8, 256, 8, 128, 1024, True, "uniform"),
    3: Workload(3, "prefill_4096x7168", 4096, 7168, 8, 256, 8, 4096, 4096, True,
                "group_limited", num_groups=8, topk_groups=4),
    4: Workload(4, "large_16384x7168", 16384, 7168, 6, 256, 8, 16384, 16384, False, "uniform"),
    5: Workload(5, "skewed_4096x4096", 4096, 4096, 6, 64, 64, 4096, 4096, True, "zipf",
                mask_fraction=0.1, zipf_s=1.2),
}


def bf16_bits(values_f32: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) of float32 values, via torch's CPU cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(values_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _softmax_f32(logits: np.ndarray) -> np.ndarray:
    z = logits.astype(np.float64)
    z = np.exp(z - z.max(axis=1, keepdims=True))
    return (z / z.sum(axis=1, keepdims=True)).astype(np.float32)


def _uniform_routing(rng, n, e, k):
    return np.argsort(rng.random((n, e)), axis=1)[:, :k].astype(np.int64)


def _group_limited_routing(rng, n, e, k, groups, topk_groups):
    s = rng.standard_normal((n, e), dtype=np.float32)
    # a group's score: binary32 sum of its experts' scores in ascending expert
    # index, from +0 (a fixed order, so every consumer ranks groups alike)
    per = s.reshape(n, groups, e // groups)
    gscore = np.zeros((n, groups), dtype=np.float32)
    for i in range(e // groups):
        gscore = gscore + per[:, :, i]
    top_groups = np.argsort(-gscore, axis=1, kind="stable")[:, :topk_groups]
    allowed = np.zeros((n, groups), dtype=bool)
    np.put_along_axis(allowed, top_groups, True, axis=1)
    cand = np.repeat(allowed, e // groups, axis=1)
    masked = np.where(cand, s, -np.inf)
    idx = np.argsort(-masked, axis=1, kind="stable")[:, :k].astype(np.int64)
    sel = np.take_along_axis(s, idx, axis=1).astype(np.float64)
    sig = 1.0 / (1.0 + np.exp(-sel))
    w = (sig / sig.sum(axis=1, keepdims=True)).astype(np.float32)
    return idx, w, s


def _zipf_routing(rng, n, e, k, s_exp):
    p = (np.arange(1, e + 1, dtype=np.float64)) ** (-s_exp)
    p /= p.sum()
    keys = np.log(p)[None, :] + rng.gumbel(size=(n, e))
    return np.argsort(-keys, axis=1, kind="stable")[:, :k].astype(np.int64)


def make_inputs(w: Workload, seed: Optional[int] = None, with_expert_rows: bool = False) -> dict:
    """Draw one batch for workload ``w``.

    Returns a dict with ``x_bits`` (uint16 [N, H], bf16 patterns),
    ``topk_idx`` (int64 [N, K], -1 = masked), ``topk_weights`` (float32
    [N, K]), ``num_valid`` (number of entries that are not -1), for
    group-limited routing ``router_scores`` (float32 [N, E], the scores the
    routing was drawn from) and, when
    ``with_expert_rows``, ``expert_rows`` (uint16 [P, H], one bf16 row per
    valid entry in (t, k) order)."""
    rng = np.random.default_rng(1000 + w.wid if seed is None else seed)
    n, h, k, e = w.num_tokens, w.hidden, w.num_topk, w.num_experts
    x_bits = bf16_bits(rng.standard_normal((n, h), dtype=np.float32))
    if w.routing == "uniform":
        topk_idx = _uniform_routing(rng, n, e, k)
        weights = _softmax_f32(rng.standard_normal((n, k), dtype=np.float32))
    elif w.routing == "group_limited":
        topk_idx, weights, scores = _group_limited_routing(rng, n, e, k, w.num_groups,
                                                           w.topk_groups)
    elif w.routing == "zipf":
        topk_idx = _zipf_routing(rng, n, e, k, w.zipf_s)
        weights = _softmax_f32(rng.standard_normal((n, k), dtype=np.float32))
    else:
        raise ValueError(f"unknown routing {w.routing!r}")
    if w.mask_fraction > 0.0:
        n_mask = int(np.floor(w.mask_fraction * n * k))
        flat = topk_idx.reshape(-1)
        flat[rng.permutation(n * k)[:n_mask]] = -1
    out = {
        "x_bits": np.ascontiguousarray(x_bits),
        "topk_idx": np.ascontiguousarray(topk_idx),
        "topk_weights": np.ascontiguousarray(weights),
        "num_valid": int((topk_idx >= 0).sum()),
    }
    if w.routing == "group_limited":
        out["router_scores"] = scores
    if with_expert_rows:
        out["expert_rows"] = bf16_bits(rng.standard_normal((out["num_valid"], h), dtype=np.float32))
    return out
