"""The bench's host-side arithmetic, without a GPU: the algorithmic bytes
behind every GB/s figure and roofline fraction, and the one-GPU guard.

The expected byte counts are worked out by hand per workload from what each
step must move (read topk_idx, write the slots and counts; read x once and
write a row, a source index and the scales per valid entry; read one expert
row per valid entry and write one output row per token), using the seeded
generator's entry counts: every entry is valid except in the skewed workload,
where exactly floor(0.1 * N * K) entries are masked."""
import subprocess
import sys
import os

import pytest

import bench
from combine_ep_layout_02_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# workload id -> (valid entries P, layout bytes, pack bytes, combine bytes)
EXPECTED = {
    # 64 x 256, K 2, E 16 / R 4, BF16: layout 12*128 + 5*256 + 4*(32+4+1)
    1: (128, 2_964, 100_352, 100_352),
    # 128 x 7168, K 8, E 256 / R 8, FP8: per entry 7168 + 4 + 56*4 = 7396 B
    2: (1_024, 19_492, 9_420_800, 16_531_456),
    # 4096 x 7168, K 8, E 256 / R 8, FP8 (the headline workload)
    3: (32_768, 559_140, 301_465_600, 529_006_592),
    # 16384 x 7168, K 6, E 256 / R 8, BF16
    4: (98_304, 1_837_092, 1_645_740_032, 1_645_740_032),
    # 4096 x 4096, K 6, E 64 / R 64, FP8, 2457 entries masked
    5: (22_119, 1_606_404, 127_368_476, 215_146_496),
}


@pytest.mark.parametrize("wid", sorted(EXPECTED))
def test_algorithmic_bytes_per_workload(wid):
    w = W.WORKLOADS[wid]
    P, lay, pack, comb = EXPECTED[wid]
    got = bench.algorithmic_bytes(w.num_tokens, w.hidden, w.num_topk, w.num_experts, w.num_ranks,
                                  P, w.use_fp8)
    assert got == {"layout": lay, "dispatch": pack, "combine": comb,
                   "total": lay + pack + comb}


def test_entry_counts_match_the_generator():
    """The P of the table is what the generator draws (routing recipe at
    full N; the hidden size does not change the routing's entry count)."""
    for wid, (P, *_rest) in EXPECTED.items():
        w = W.WORKLOADS[wid]
        inp = W.make_inputs(w.scaled(w.num_tokens, 128))
        assert inp["num_valid"] == P, wid


def test_scale_format_bytes():
    """UE8M0 packs four 1-byte exponents per 32-bit word: at H = 7168 the 56
    fp32 scales per row (224 B) become 14 words (56 B)."""
    n, h, k, e, r, p = 4096, 7168, 8, 256, 8, 32_768
    fp32 = bench.algorithmic_bytes(n, h, k, e, r, p, True, 0)["dispatch"]
    ue8m0 = bench.algorithmic_bytes(n, h, k, e, r, p, True, 2)["dispatch"]
    assert fp32 - ue8m0 == p * (224 - 56)
    assert bench.algorithmic_bytes(n, h, k, e, r, p, True, 1)["dispatch"] == fp32


def test_receive_layout_bytes_by_hand():
    """Normal mode and expand layout at a small shape: N 4, H 256, K 2, R 2,
    5 valid entries sent as 3 (token, rank) rows, 2 padding rows, FP8."""
    n, h, k, r, p, rows, pad = 4, 256, 2, 2, 5, 3, 2
    row = 256 + 4 * 2 + 4  # FP8 payload, two fp32 scales, the source index
    got = bench.receive_layout_bytes(n, h, k, r, p, rows, pad, True)
    assert got["dispatch_normal"] == 2 * n * h + 4 * n * r + 12 * n * k + rows * (row + 12 * k)
    assert got["combine_normal"] == 4 * n * r + rows * (2 * h + 4 * k) + n * (2 * h + 4 * k)
    assert got["dispatch_expand"] == 2 * n * h + 12 * n * k + (p + pad) * row
    assert got["combine_expand"] == 2 * p * h + 16 * n * k + 2 * n * h


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode != 0
    assert "one GPU" in res.stderr
    assert res.stdout.strip() == ""


def test_profile_grid_sizes():
    """The grid sizes the profile summaries match kernels by: pack and
    combine one 64-lane wave per (token, 1024-channel chunk) in 256-thread
    blocks; the layout 256 tokens per block plus the totals block; the fused
    layout + pack one block per token plus the totals block, 512 threads up
    to 256 tokens and 256 above."""
    assert bench._grid_threads(4096, 7168, "pack") == 4096 * 7 * 64
    assert bench._grid_threads(128, 7168, "combine") == 128 * 7 * 64
    assert bench._grid_threads(130, 1000, "pack") == -(-130 // 4) * 256
    assert bench._grid_threads(4096, 7168, "layout_count") == 16 * 256
    assert bench._grid_threads(4096, 7168, "layout_assign") == 17 * 256
    assert bench._grid_threads(128, 7168, "layout_assign") == 256
    assert bench._grid_threads(128, 7168, "fused") == 129 * 512
    assert bench._grid_threads(600, 7168, "fused") == 601 * 256


def test_cpu_baseline_times_each_phase():
    """The CPU baseline runs the oracle's timed path per workload: three
    phase figures, their sum, the GB/s they give, the CPU model and one
    thread."""
    cb = bench.cpu_baseline(2, lambda m: None, workloads=(1,))
    ph = cb["per_workload"]["tiny_64x256"]
    assert ph["runs"] == 2 and min(ph["layout_ms"], ph["pack_ms"], ph["combine_ms"]) >= 0
    assert abs(ph["step_ms"] - (ph["layout_ms"] + ph["pack_ms"] + ph["combine_ms"])) < 0.01
    assert cb["value"] == ph["gbps"] > 0 and cb["cores"] == 1 and cb["threads"] == 1
    assert cb["cpu_model"] and cb["kind"] == "oracle"
