"""GPU parity of the top-k combine across batch sizes.

The library runs one wave per (token, chunk) item when one round of resident
waves covers every item, and otherwise a grid that is resident all at once
with 8 or 14 items per wave, whose outputs are stored after the wave's last
read; past 14 items per resident wave it goes back to one wave per item.
Which one runs depends on the batch size and on the occupancy the device
reports, so these sizes (H = 7,168, top-8 of 256 experts; the two largest
with 16 experts to keep the expert buffer small, one with top-6) step across
every boundary on an MI355X.  Each size is
compared with the oracle element by element, with masked entries,
out-of-range ids and, on three sizes, the epilogue bias; bit-identical is
expected (the tolerance of the other combine tests is the bar) and the
status bits must match.
"""
import numpy as np
import pytest

import oracle
import pins
from combine_ep_layout_02_amd import ep
from combine_ep_layout_02_amd import workloads as W
from gpu_helpers import LayoutRun, place_expert_rows, run_combine, say

pytestmark = pytest.mark.gpu

SIZES = [(700, 8, 256), (800, 8, 256), (1500, 8, 256), (2600, 8, 256), (3000, 8, 256),
         (3600, 8, 256), (4100, 8, 256), (9000, 8, 16), (12000, 6, 16)]
WITH_BIAS = (800, 3000, 9000)


@pytest.fixture(scope="module")
def o():
    return oracle.get()


@pytest.mark.parametrize("N,K,E", SIZES, ids=[f"{n}-top{k}-of-{e}" for n, k, e in SIZES])
def test_combine_across_batch_sizes(o, N, K, E):
    H, R = 7168, 8
    rng = np.random.default_rng(N)
    idx = np.argsort(rng.random((N, E), dtype=np.float32), axis=1)[:, :K].astype(np.int64)
    idx[rng.random((N, K)) < 0.05] = -1
    bad = rng.permutation(N * K)[:5]
    idx.reshape(-1)[bad] = E + 3
    weights = rng.random((N, K), dtype=np.float32)
    shape = ep.make_shape(N, H, K, E, R, N, N, False)
    say(f"ep_combine N={N} H={H} K={K} E={E} bias={N in WITH_BIAS}")
    run = LayoutRun(shape, idx)
    lay = run.numpy()
    valid = (idx >= 0) & (idx < E)
    masked = np.where(valid, idx, -1)
    rows = W.bf16_bits(rng.standard_normal((int(valid.sum()), H), dtype=np.float32))
    y = place_expert_rows(rows, masked, lay["expert_slot"], E, N, H)
    s_or = max(1, int(lay["num_tokens_per_expert"].max()))
    y_or = pins.place_rows(rows, masked, lay["expert_slot"], E, s_or)
    bias = None
    if N in WITH_BIAS:
        bias = W.bf16_bits(rng.standard_normal((N, H), dtype=np.float32))
    got, st = run_combine(shape, y, run.topk_idx, weights, run.expert_slot, bias=bias)
    want, st_or = o.combine(y_or, idx, weights, lay["expert_slot"], E, s_or, bias=bias)
    assert st == st_or, (N, st, st_or)
    assert st & ep.EP_STATUS_BAD_EXPERT_ID
    pins.assert_combine_close(got, pins.bf16_to_f64(want), f"combine N={N}")
    ndiff = int((got != want).sum())
    assert ndiff == 0, f"N={N}: within tolerance but {ndiff} elements not bit-identical"
