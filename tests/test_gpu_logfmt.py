"""GPU parity of the LogFMT combine payload against the CPU oracle.

Bar: the encoder's logarithm, codes and headers are bit-exact (every binary32
step of the encoding is the same operation on both sides).  The combine of
LogFMT rows is within 1 bf16 ulp or 8e-3 relative of the oracle's, plus an
absolute allowance of (K + 4) * 2^-23 * sum_k |w_k y_k|: the device's fp32
exponential may give each decoded value y_k one ulp (2^-23 relative) away
from the oracle's correctly rounded one, each product then differs by at
most that, and the K fused multiply-adds of the chain may round differently
by 2^-24 of the running sum each; where the terms cancel, that absolute
difference dominates the small result.  Outputs and code buffers start poisoned, so an element the
kernels fail to write is caught, and rows the routing does not reference
must keep the poison.
"""
import numpy as np
import pytest
import torch

import oracle
import pins
from combine_ep_layout_02_amd import ep
from combine_ep_layout_02_amd import workloads as W
from gpu_helpers import LayoutRun, dev, host, place_expert_rows, say, status_bits, written_rows

pytestmark = pytest.mark.gpu

POISON_CODE = 0xEE
POISON_HEADER = np.float32(-12345.0)


@pytest.fixture(scope="module")
def o():
    return oracle.get()


def test_log2_probe_every_bf16(o):
    """The encoder's rounded log2 on every finite nonzero bf16 input (both
    signs) equals the oracle's, which its own pin holds to the correctly
    rounded value; zeros give -inf."""
    mags = np.arange(1, 0x7F80, dtype=np.uint16)
    bits = np.concatenate([mags, mags | 0x8000, np.array([0, 0x8000], np.uint16)])
    out = torch.full((bits.size,), float("nan"), dtype=torch.float32, device="cuda")
    ep.ep_probe_log2_bf16(dev(bits), out)
    torch.cuda.synchronize()
    got = host(out)
    want = o.log2_rn(pins.bf16_to_f64(mags).astype(np.float32))
    n = mags.size
    for part in (got[:n], got[n:2 * n]):
        bad = np.nonzero(part.view(np.uint32) != want.view(np.uint32))[0]
        assert bad.size == 0, (mags[bad[:4]], part[bad[:4]], want[bad[:4]])
    assert np.isneginf(got[-2:]).all()


def rows_of_kind(rng, P, H, kind):
    if kind == "normal":
        x = rng.standard_normal((P, H))
    elif kind == "wide":
        x = rng.standard_normal((P, H)) * np.exp2(rng.uniform(-60, 60, size=(P, H)))
    elif kind == "zeros":
        x = rng.standard_normal((P, H))
        x[rng.random((P, H)) < 0.4] = 0.0
        x[: max(P // 7, 1), :128] = 0.0  # whole zero blocks
        x[1::11, 128:256] = 3.0          # blocks of one repeated value: lo == hi
    elif kind == "extremes":
        x = rng.standard_normal((P, H)) * rng.choice([2.0 ** -130, 2.0 ** 120, 1.0], size=(P, 1))
    else:
        raise ValueError(kind)
    return W.bf16_bits(x.astype(np.float32))


def run_logfmt(o, shape, idx, wts, rows, name, bias=None, sample_tokens=None):
    """Encode + combine on the GPU against the oracle; returns the number of
    combine elements that differ at all (expected small)."""
    E, S, H, N, K = shape.num_experts, shape.expert_capacity, shape.hidden, shape.num_tokens, shape.num_topk
    say(f"logfmt {name} N={N} H={H} K={K} E={E} S={S}")
    run = LayoutRun(shape, idx)
    lay = run.numpy()
    placed = np.where((idx >= 0) & (idx < E), idx, -1)  # bad ids have no row
    y = place_expert_rows(rows, placed, lay["expert_slot"], E, S, H)
    codes = torch.full((E, S, H), POISON_CODE, dtype=torch.uint8, device="cuda")
    headers = torch.full((E, S, H // 128, 2), float(POISON_HEADER), dtype=torch.float32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ep.ep_logfmt_encode(shape, y, run.topk_idx, run.expert_slot, codes, headers, status)
    out = torch.full((N, H), -1, dtype=torch.int16, device="cuda")
    w_dev = dev(wts)
    b_dev = None if bias is None else dev(bias)
    ep.ep_combine_logfmt(shape, codes, headers, run.topk_idx, w_dev, run.expert_slot, out, status,
                         bias=b_dev)
    torch.cuda.synchronize()
    assert status_bits(status) == lay["status"]
    counts = lay["num_tokens_per_expert"]
    wr = written_rows(counts, S)
    # codes and headers of every referenced row, against the oracle's encoding
    # of the same bf16 rows (all of them, or a sample at full size)
    pick = wr if sample_tokens is None else np.sort(
        np.random.default_rng(N).choice(wr, size=min(wr.size, 3000), replace=False))
    idx_t = torch.from_numpy(pick).cuda()
    y_rows = host(y.reshape(E * S, H).index_select(0, idx_t))
    want_c, want_h = o.logfmt_encode(y_rows)
    got_c = host(codes.reshape(E * S, H).index_select(0, idx_t))
    got_h = host(headers.reshape(E * S, H // 128, 2).index_select(0, idx_t))
    bad = np.nonzero((got_c != want_c).any(axis=1))[0]
    assert bad.size == 0, (name, "codes differ in row", pick[bad[:3]])
    assert np.array_equal(got_h.view(np.uint32), want_h.view(np.uint32)), (name, "headers differ")
    # rows no entry references keep the poison
    mask = np.zeros(E * S, bool)
    mask[wr] = True
    unref = np.nonzero(~mask)[0][:20000]
    if unref.size:
        u = torch.from_numpy(unref).cuda()
        assert bool((codes.reshape(E * S, H).index_select(0, u) == POISON_CODE).all())
        assert bool((headers.reshape(E * S, -1).index_select(0, u) == float(POISON_HEADER)).all())
    # the combine, for every token or a sample of them, from the oracle's own
    # encoding of the rows those tokens reference
    toks = np.arange(N) if sample_tokens is None else np.sort(
        np.random.default_rng(N + 1).choice(N, size=min(N, sample_tokens), replace=False))
    sub_idx, sub_w = idx[toks], wts[toks]
    sub_slot = lay["expert_slot"][toks]
    valid = (sub_idx >= 0) & (sub_idx < E)  # ids outside [-1, E) count as masked
    keep = valid & (sub_slot < S)
    rows_needed = (sub_idx[keep].astype(np.int64) * S + sub_slot[keep]).astype(np.int64)
    uniq, inv = np.unique(rows_needed, return_inverse=True)
    yr = host(y.reshape(E * S, H).index_select(0, torch.from_numpy(uniq).cuda()))
    c_u, h_u = o.logfmt_encode(yr)
    # the GPU's codes and headers of exactly these rows must be the oracle's
    g_c = host(codes.reshape(E * S, H).index_select(0, torch.from_numpy(uniq).cuda()))
    g_h = host(headers.reshape(E * S, H // 128, 2).index_select(0, torch.from_numpy(uniq).cuda()))
    badr = np.nonzero((g_c != c_u).any(axis=1))[0]
    assert badr.size == 0, (name, "codes of combined rows differ", uniq[badr[:3]],
                            [np.nonzero(g_c[i] != c_u[i])[0][:4] for i in badr[:3]])
    assert np.array_equal(g_h.view(np.uint32), h_u.view(np.uint32)), (name, "headers of combined rows")
    # a compact [len(uniq) + 1, 1, H] buffer (row i = uniq[i]); masked entries stay -1
    c_buf = np.concatenate([c_u, np.zeros((1, H), np.uint8)])[:, None, :]
    h_buf = np.concatenate([h_u, np.zeros((1, H // 128, 2), np.float32)])[:, None, :, :]
    cidx = np.full(sub_idx.shape, -1, np.int64)
    cidx[keep] = inv
    cslot = np.zeros(sub_idx.shape, np.int32)
    cb = None if bias is None else bias[toks]
    want, st = o.combine_logfmt(c_buf, h_buf, cidx, sub_w, cslot, len(uniq) + 1, 1, bias=cb)
    got = host(out)[toks]
    ref = pins.bf16_to_f64(want)
    dec = np.abs(o.logfmt_decode(c_u, h_u).astype(np.float64))
    absum = np.zeros((len(toks), H))
    for k in range(K):
        m = cidx[:, k] >= 0
        absum[m] += np.abs(sub_w[m, k].astype(np.float64))[:, None] * dec[cidx[m, k]]
    if bias is not None:
        absum += np.abs(pins.bf16_to_f64(bias[toks]))
    slack = (K + 4) * 2.0 ** -23 * absum
    pins.assert_combine_close(got, ref, f"{name} combine_logfmt", abs_slack=slack)
    return int((got != want).sum())


CASES = [  # (workload, N, H, kind)
    (1, 64, 256, "normal"),
    (2, 128, 1024, "wide"),
    (3, 300, 896, "zeros"),
    (4, 200, 384, "extremes"),
    (5, 250, 512, "zeros"),
]


@pytest.mark.parametrize("wid,N,H,kind", CASES)
def test_logfmt_small(o, wid, N, H, kind):
    w = W.WORKLOADS[wid].scaled(N, H)
    inp = W.make_inputs(w, seed=6000 + wid)
    shape = ep.shape_of(w)
    rng = np.random.default_rng(wid)
    rows = rows_of_kind(rng, inp["num_valid"], H, kind)
    diff = run_logfmt(o, shape, inp["topk_idx"], inp["topk_weights"], rows, f"{w.name} {kind}")
    say(f"  combine elements not bit-identical: {diff}")


def test_logfmt_bias_masked_and_bad_ids(o):
    """A shared-expert bias in the epilogue, masked entries, an id outside
    [-1, E) (treated as masked, reported) and K = 3 (the 4-entry batch)."""
    N, H, K, E, R = 150, 512, 3, 16, 4
    rng = np.random.default_rng(3)
    idx = np.argsort(rng.random((N, E)), axis=1)[:, :K].astype(np.int64)
    idx[rng.random((N, K)) < 0.2] = -1
    idx[7, 1] = E + 5
    wts = rng.random((N, K)).astype(np.float32)
    shape = ep.make_shape(N, H, K, E, R, N, N, False)
    clean = np.where(idx >= E, -1, idx)
    rows = rows_of_kind(rng, int((clean >= 0).sum()), H, "normal")
    bias = W.bf16_bits(rng.standard_normal((N, H)).astype(np.float32))
    run_logfmt(o, shape, idx, wts, rows, "bias + masked + bad id", bias=bias)


def test_logfmt_large_batch_with_bias(o):
    """A batch large enough for the table encoder (4,096 tokens x 2,560
    channels: 12,288 items), with a bias, masked entries and a partial last
    chunk (2,560 = 2 x 1,024 + 512)."""
    w = W.WORKLOADS[3].scaled(4096, 2560)
    inp = W.make_inputs(w, seed=77)
    idx = inp["topk_idx"].copy()
    rng = np.random.default_rng(78)
    idx[rng.random(idx.shape) < 0.1] = -1
    rows = rows_of_kind(rng, int((idx >= 0).sum()), w.hidden, "zeros")
    bias = W.bf16_bits(rng.standard_normal((w.num_tokens, w.hidden)).astype(np.float32))
    run_logfmt(o, ep.shape_of(w), idx, inp["topk_weights"], rows, "large batch + bias",
               bias=bias, sample_tokens=300)


@pytest.mark.parametrize("kind", ["wide", "extremes", "zeros"])
def test_logfmt_table_encoder_special_values(o, kind):
    """Rows spanning 2^-60..2^60, rows scaled to subnormal and huge
    magnitudes, and rows with zero channels and whole zero or constant
    blocks, at a batch (2,048 tokens x 2,048 channels: 4,096 items) that
    takes the table encoder: codes and headers bit-exact, as the per-item
    encoder's are on the small cases."""
    w = W.WORKLOADS[3].scaled(2048, 2048)
    inp = W.make_inputs(w, seed=91)
    rng = np.random.default_rng(92)
    rows = rows_of_kind(rng, inp["num_valid"], w.hidden, kind)
    run_logfmt(o, ep.shape_of(w), inp["topk_idx"], inp["topk_weights"], rows,
               f"table encoder {kind}", sample_tokens=300)


def test_logfmt_full_size_prefill(o):
    """The prefill workload at full size (4,096 x 7,168, top-8 of 256): codes
    and headers of 3,000 sampled rows bit-exact, the combine of 256 sampled
    tokens within the bar, rows nobody references untouched."""
    w = W.WORKLOADS[3]
    inp = W.make_inputs(w, with_expert_rows=True)
    run_logfmt(o, ep.shape_of(w), inp["topk_idx"], inp["topk_weights"], inp["expert_rows"],
               w.name, sample_tokens=256)


def test_logfmt_decode_shape(o):
    """The decode workload (128 x 7,168, S = 1,024 rows per expert) in full."""
    w = W.WORKLOADS[2]
    inp = W.make_inputs(w, with_expert_rows=True)
    run_logfmt(o, ep.shape_of(w), inp["topk_idx"], inp["topk_weights"], inp["expert_rows"], w.name)


def test_logfmt_rejects_hidden_not_multiple_of_128():
    shape = ep.make_shape(4, 200, 2, 8, 2, 4, 4, False)
    t = lambda n, dt: torch.zeros(n, dtype=dt, device="cuda")
    with pytest.raises(ep.EpError) as err:
        ep.ep_logfmt_encode(shape, t(8 * 4 * 200, torch.int16), t(8, torch.int64),
                            t(8, torch.int32), t(8 * 4 * 200, torch.uint8), t(8 * 4 * 4, torch.float32))
    assert err.value.code == ep.EP_ERR_SHAPE
