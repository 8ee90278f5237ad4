"""ep_layout_noalloc: the dispatch layout on the library's static per-device
scratch, for callers that cannot allocate device memory.  Its outputs must
equal ep_layout's (caller workspace) bit for bit, call after call, on the one
scratch array that every call on the GPU shares and that keeps the previous
call's contents.

Each call runs on poisoned outputs (an element left unwritten is caught), on
the same routing as an ep_layout call with a poisoned workspace, and the
result is also held against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
from combine_ep_layout_02_amd import ep
from combine_ep_layout_02_amd import workloads as W
from gpu_helpers import POISON_I32, POISON_U8, LayoutRun, dev, host, say, status_bits

pytestmark = pytest.mark.gpu

LAYOUT_KEYS = ("num_tokens_per_rank", "num_tokens_per_expert", "is_token_in_rank", "expert_slot",
               "rank_slot", "expert_offset")


def noalloc_layout(shape, topk_idx_dev, stream=None):
    """One ep_layout_noalloc call on poisoned outputs -> numpy dict."""
    N, K, E, R = shape.num_tokens, shape.num_topk, shape.num_experts, shape.num_ranks
    full = lambda n, v, dt: torch.full((n,), v, dtype=dt, device="cuda")
    out = {
        "num_tokens_per_rank": full(R, POISON_I32, torch.int32),
        "num_tokens_per_expert": full(E, POISON_I32, torch.int32),
        "is_token_in_rank": full(N * R, POISON_U8, torch.uint8).view(N, R),
        "expert_slot": full(N * K, POISON_I32, torch.int32).view(N, K),
        "rank_slot": full(N * R, POISON_I32, torch.int32).view(N, R),
        "expert_offset": full(E + 1, POISON_I32, torch.int32),
    }
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    if stream is not None:
        # the fills above ran on the current stream: order them before the call
        stream.wait_stream(torch.cuda.current_stream())
    ep.ep_layout_noalloc(shape, topk_idx_dev, out["num_tokens_per_rank"],
                         out["num_tokens_per_expert"], out["is_token_in_rank"], out["expert_slot"],
                         out["rank_slot"], out["expert_offset"], status, stream=stream)
    torch.cuda.synchronize()
    got = {k: host(v) for k, v in out.items()}
    got["status"] = status_bits(status)
    return got


def routing(wid, num_tokens):
    w = W.WORKLOADS[wid].scaled(num_tokens, hidden=128)
    inp = W.make_inputs(w, seed=5000 + wid * 7 + num_tokens)
    return ep.shape_of(w), inp["topk_idx"]


# each call uses fewer histogram rows than the one before (the last none), so
# a call that read a row its own count kernel did not write would see the
# previous call's contents
SEQUENCE = [(4, 16384), (4, 12000), (3, 4096), (5, 1000), (3, 300), (2, 128)]


def layout_scratch_bytes(shape):
    """Bytes of ep_layout's histogram rows (include/ep.h: B * round_up(E + R,
    4) * 4, B = ceil(N / 256), none for a single block)."""
    blocks = -(-shape.num_tokens // 256)
    return 0 if blocks <= 1 else blocks * (-(-(shape.num_experts + shape.num_ranks) // 4) * 4) * 4


@pytest.mark.parametrize("stream_kind", ["current", "side"])
def test_noalloc_matches_ep_layout_call_after_call(stream_kind):
    o = oracle.get()
    stream = None if stream_kind == "current" else torch.cuda.Stream()
    for wid, n in SEQUENCE:
        shape, idx = routing(wid, n)
        need = layout_scratch_bytes(shape)
        assert need <= ep.EP_NOALLOC_SCRATCH_BYTES
        say(f"ep_layout_noalloc workload {wid} N={n} K={shape.num_topk} E={shape.num_experts} "
            f"R={shape.num_ranks} scratch bytes used {need} stream {stream_kind}")
        idx_dev = dev(idx)
        got = noalloc_layout(shape, idx_dev, stream=stream)
        ref = LayoutRun(shape, idx).numpy()  # ep_layout with a poisoned caller workspace
        want = o.layout(idx, shape.num_experts, shape.num_ranks)
        for key in LAYOUT_KEYS:
            assert np.array_equal(got[key], ref[key]), (wid, n, key)
            assert np.array_equal(got[key], want[key]), (wid, n, key)
        assert got["status"] == ref["status"] == 0


def test_noalloc_rejects_a_shape_beyond_its_scratch():
    # 300,000 tokens at E = 256, R = 8 need 1,172 histogram rows of 1,056 B
    shape = ep.make_shape(300_000, 128, 8, 256, 8, 300_000, 300_000, False)
    assert layout_scratch_bytes(shape) > ep.EP_NOALLOC_SCRATCH_BYTES
    t = lambda n, dt: torch.empty(n, dtype=dt, device="cuda")
    with pytest.raises(ep.EpError) as err:
        ep.ep_layout_noalloc(shape, t(300_000 * 8, torch.int64), t(8, torch.int32),
                             t(256, torch.int32), t(300_000 * 8, torch.uint8),
                             t(300_000 * 8, torch.int32), t(300_000 * 8, torch.int32),
                             t(257, torch.int32))
    assert err.value.code == ep.EP_ERR_SCRATCH
