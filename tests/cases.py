"""Small seeded cases shared by the CPU pin tests and the GPU parity tests.

Every case comes from ``combine_ep_layout_02_amd.workloads`` (the seeded
input generator); nothing here computes any part of the method."""
from __future__ import annotations

import numpy as np

from combine_ep_layout_02_amd import workloads as W


def scaled_inputs(wid: int, num_tokens: int, hidden: int, seed: int | None = None):
    """Workload ``wid``'s recipe at a reduced size: (workload, inputs)."""
    w = W.WORKLOADS[wid].scaled(num_tokens, hidden)
    return w, W.make_inputs(w, seed=seed, with_expert_rows=True)


def small_cases():
    """(workload, inputs) pairs spanning all five recipes at sizes the oracle
    finishes in well under a second, with ragged token counts."""
    return [
        (W.WORKLOADS[1], W.make_inputs(W.WORKLOADS[1], with_expert_rows=True)),
        scaled_inputs(2, 40, 256),
        scaled_inputs(3, 70, 384),
        scaled_inputs(4, 90, 136),
        scaled_inputs(5, 100, 256),
    ]


def with_dead_tokens(inp: dict, every: int = 7) -> dict:
    """A copy of ``inp`` where every ``every``-th token has all entries
    masked (-1)."""
    out = dict(inp)
    idx = inp["topk_idx"].copy()
    idx[::every] = -1
    out["topk_idx"] = idx
    out["num_valid"] = int((idx >= 0).sum())
    out.pop("expert_rows", None)
    return out
